"""Python binding of libsmla.so -- sparse MLA decode with split-K over the
top-k list on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/smla.h).  torch supplies device memory and
the stream; there is no CPU fallback.  The library is loaded on first use
(so that the package's build module can run before it exists): any call
without the built library raises ImportError.

Functions carry the C names: smla_plan_nsplit, smla_plan_nsplit_cus,
smla_workspace_bytes, smla_workspace_lse_offset, smla_decode, smla_decode_fused,
smla_fused_in_launch, smla_set_merge_polls, smla_decode_paged, smla_decode_dense,
smla_plan_nsplit_dense, smla_split, smla_combine, smla_topk, smla_topk_workspace_bytes,
smla_set_topk_min_chunks, smla_status_str.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla.so")

ROW = 576
DV = 512
MAX_NSPLIT = 1024

STATUS = {0: "SMLA_OK", -1: "SMLA_ERR_NULL", -2: "SMLA_ERR_DIM", -3: "SMLA_ERR_NSPLIT",
          -4: "SMLA_ERR_WORKSPACE", -5: "SMLA_ERR_ALIGN", -6: "SMLA_ERR_DEVICE",
          -7: "SMLA_ERR_LAUNCH"}


class SmlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({smla_status_str(code)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_mla_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    lib.smla_plan_nsplit.argtypes = [i32, i32, i32, i32]
    lib.smla_plan_nsplit.restype = i32
    lib.smla_plan_nsplit_cus.argtypes = [i32, i32, i32, i32, i32]
    lib.smla_plan_nsplit_cus.restype = i32
    lib.smla_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.smla_workspace_bytes.restype = sz
    lib.smla_workspace_lse_offset.argtypes = [i32, i32, i32, i32]
    lib.smla_workspace_lse_offset.restype = sz
    lib.smla_fused_in_launch.argtypes = [i32, i32, i32, i32]
    lib.smla_fused_in_launch.restype = i32
    lib.smla_set_merge_polls.argtypes = [i32]
    lib.smla_set_merge_polls.restype = i32
    call = [vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i64, vp, sz, vp]
    lib.smla_decode.argtypes = call
    lib.smla_decode.restype = i32
    lib.smla_decode_fused.argtypes = call
    lib.smla_decode_fused.restype = i32
    lib.smla_split.argtypes = call
    lib.smla_split.restype = i32
    lib.smla_decode_paged.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, f32, i32, i32, i32, i32,
                                      i32, i64, vp, sz, vp]
    lib.smla_decode_paged.restype = i32
    lib.smla_decode_dense.argtypes = [vp, vp, vp, i32, i32, vp, i32, vp, vp, f32, i32, i32, i32,
                                      i32, i64, vp, sz, vp]
    lib.smla_decode_dense.restype = i32
    lib.smla_plan_nsplit_dense.argtypes = [i32, i32, i32, i32]
    lib.smla_plan_nsplit_dense.restype = i32
    lib.smla_combine.argtypes = [vp, vp, vp, vp, i32, i32, i32, vp]
    lib.smla_combine.restype = i32
    lib.smla_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.smla_topk.restype = i32
    lib.smla_topk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.smla_topk_workspace_bytes.restype = sz
    lib.smla_set_topk_min_chunks.argtypes = [i32]
    lib.smla_set_topk_min_chunks.restype = i32
    lib.smla_status_str.argtypes = [i32]
    lib.smla_status_str.restype = ctypes.c_char_p
    return lib


_handle = None


def _lib_handle() -> ctypes.CDLL:
    global _handle
    if _handle is None:
        _handle = _load()
    return _handle


def __getattr__(name):
    # `lib`: the raw ctypes handle (tests call the C ABI through it)
    if name == "lib":
        return _lib_handle()
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")


def smla_status_str(status: int) -> str:
    return _lib_handle().smla_status_str(int(status)).decode()


def smla_plan_nsplit(batch: int, q_len: int, heads: int, topk: int) -> int:
    r = _lib_handle().smla_plan_nsplit(batch, q_len, heads, topk)
    if r < 1:
        raise SmlaError(r, "smla_plan_nsplit")
    return r


def smla_plan_nsplit_cus(cus: int, batch: int, q_len: int, heads: int, topk: int) -> int:
    r = _lib_handle().smla_plan_nsplit_cus(cus, batch, q_len, heads, topk)
    if r < 1:
        raise SmlaError(r, "smla_plan_nsplit_cus")
    return r


def smla_workspace_bytes(batch: int, q_len: int, heads: int, nsplit: int) -> int:
    return int(_lib_handle().smla_workspace_bytes(batch, q_len, heads, nsplit))


def smla_workspace_lse_offset(batch: int, q_len: int, heads: int, nsplit: int) -> int:
    return int(_lib_handle().smla_workspace_lse_offset(batch, q_len, heads, nsplit))


def smla_set_merge_polls(polls: int) -> int:
    """Bound on a waiting workgroup's polls in the single-launch merge
    (0 = the last arriver merges the whole unit).  Returns the previous value."""
    r = _lib_handle().smla_set_merge_polls(polls)
    if r < 0:
        raise SmlaError(r, "smla_set_merge_polls")
    return r


def smla_fused_in_launch(batch: int, q_len: int, heads: int, nsplit: int) -> bool:
    """Whether smla_decode_fused of this shape merges inside the split launch."""
    r = _lib_handle().smla_fused_in_launch(batch, q_len, heads, nsplit)
    if r < 0:
        raise SmlaError(r, "smla_fused_in_launch")
    return bool(r)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _shape(q: torch.Tensor, topk_idx: torch.Tensor):
    if q.dim() != 4 or q.shape[-1] != ROW:
        raise ValueError(f"q must be [batch, q_len, heads, {ROW}], got {tuple(q.shape)}")
    b, lq, h, _ = q.shape
    if topk_idx.dim() != 3 or tuple(topk_idx.shape[:2]) != (b, lq):
        raise ValueError(f"topk_idx must be [batch, q_len, topk], got {tuple(topk_idx.shape)}")
    return b, lq, h, topk_idx.shape[2]


def _check_tensors(q, kv_cache, topk_idx, out, lse):
    for name, t, dt in (("q", q, torch.bfloat16), ("kv_cache", kv_cache, torch.bfloat16),
                        ("topk_idx", topk_idx, torch.int32), ("out", out, torch.bfloat16),
                        ("lse", lse, torch.float32)):
        if t is None:
            continue
        if t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if kv_cache.dim() != 2 or kv_cache.shape[1] != ROW:
        raise ValueError(f"kv_cache must be [rows, {ROW}], got {tuple(kv_cache.shape)}")


WS_SYNC_BYTES = 16384  # SMLA_WS_SYNC_BYTES: the workspace's synchronisation words


def workspace(batch: int, q_len: int, heads: int, nsplit: int, device) -> torch.Tensor | None:
    """A workspace tensor of the size the call needs (None when nsplit <= 1),
    its synchronisation words zeroed as the library requires."""
    n = smla_workspace_bytes(batch, q_len, heads, nsplit)
    if not n:
        return None
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    ws[:WS_SYNC_BYTES].zero_()
    return ws


def _call(fn, name, q, kv_cache, topk_idx, out, lse, scale, nsplit, ws, stream):
    _check_tensors(q, kv_cache, topk_idx, out, lse)
    b, lq, h, k = _shape(q, topk_idx)
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit(b, lq, h, k)
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = fn(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(out), _ptr(lse), float(scale),
            int(nsplit), b, lq, h, k, kv_cache.shape[0], _ptr(ws), ws_bytes, _stream(stream))
    if rc != 0:
        raise SmlaError(rc, name)
    return nsplit, ws


def smla_decode(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int = 0,
                workspace_t=None, stream=None) -> int:
    """Sparse MLA decode into `out` [B, Lq, H, 512] bf16 and `lse` [B, Lq, H] fp32.

    nsplit 0 asks the planner.  A workspace is allocated when none is given
    and NSPLIT > 1.  Returns the NSPLIT used.
    """
    return _call(_lib_handle().smla_decode, "smla_decode", q, kv_cache, topk_idx, out, lse, scale, nsplit,
                 workspace_t, stream)[0]


def smla_decode_fused(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int = 0,
                      workspace_t=None, stream=None) -> int:
    """smla_decode with the merge inside the split launch when the shape
    allows it (smla_fused_in_launch), else exactly smla_decode.  A given
    workspace must have its first WS_SYNC_BYTES zero (workspace() does that);
    the call leaves them zero.  Returns the NSPLIT used."""
    return _call(_lib_handle().smla_decode_fused, "smla_decode_fused", q, kv_cache, topk_idx, out, lse,
                 scale, nsplit, workspace_t, stream)[0]


def smla_split(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int,
               workspace_t=None, stream=None):
    """Split kernel alone.  Returns (nsplit, workspace) -- the partials live in
    the workspace (see partials_view) when NSPLIT > 1."""
    return _call(_lib_handle().smla_split, "smla_split", q, kv_cache, topk_idx, out, lse, scale, nsplit,
                 workspace_t, stream)


def _check_table(block_table, what):
    if block_table is None:
        return 0
    if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2:
        raise ValueError(f"{what}: block_table must be a contiguous int32 [batch, max_pages] tensor")
    return block_table.shape[1]


def smla_decode_paged(q, kv_cache, block_table, page_size: int, topk_pos, out, lse, scale: float,
                      nsplit: int = 0, workspace_t=None, stream=None) -> int:
    """smla_decode with topk_pos [B, Lq, K] holding positions in each
    sequence, mapped to cache rows through block_table [B, max_pages] inside
    the kernel.  Returns the NSPLIT used."""
    _check_tensors(q, kv_cache, topk_pos, out, lse)
    b, lq, h, k = _shape(q, topk_pos)
    max_pages = _check_table(block_table, "smla_decode_paged")
    if block_table is None or block_table.shape[0] != b:
        raise ValueError("smla_decode_paged: block_table must be [batch, max_pages]")
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit(b, lq, h, k)
    ws = workspace_t
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = _lib_handle().smla_decode_paged(_ptr(q), _ptr(kv_cache), _ptr(block_table), max_pages, page_size,
                                _ptr(topk_pos), _ptr(out), _ptr(lse), float(scale), int(nsplit),
                                b, lq, h, k, kv_cache.shape[0], _ptr(ws), ws_bytes, _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_decode_paged")
    return nsplit


def smla_plan_nsplit_dense(batch: int, q_len: int, heads: int, max_ctx: int) -> int:
    r = _lib_handle().smla_plan_nsplit_dense(batch, q_len, heads, max_ctx)
    if r < 1:
        raise SmlaError(r, "smla_plan_nsplit_dense")
    return r


def dense_folds(q_len: int, heads: int, max_ctx: int) -> bool:
    """Whether smla_decode_dense runs a sequence's tokens as heads of one
    token (the rule stated in include/smla.h)."""
    return q_len > 1 and q_len * heads <= 4096 and max_ctx >= 8192


def smla_decode_dense(q, kv_cache, ctx_len, max_ctx: int, out, lse, scale: float, nsplit: int = 0,
                      block_table=None, page_size: int = 1, workspace_t=None, stream=None) -> int:
    """Dense KV-split decode: each token of sequence b attends to positions
    0 .. ctx_len[b]-1 (rows through block_table when given, else position =
    row).  Returns the NSPLIT used."""
    _check_tensors(q, kv_cache, None, out, lse)
    if q.dim() != 4 or q.shape[-1] != ROW:
        raise ValueError(f"q must be [batch, q_len, heads, {ROW}], got {tuple(q.shape)}")
    b, lq, h, _ = q.shape
    if ctx_len.dtype != torch.int32 or ctx_len.shape != (b,) or not ctx_len.is_contiguous():
        raise ValueError("smla_decode_dense: ctx_len must be a contiguous int32 [batch] tensor")
    max_pages = _check_table(block_table, "smla_decode_dense")
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit_dense(b, lq, h, max_ctx)
    ws = workspace_t
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = _lib_handle().smla_decode_dense(_ptr(q), _ptr(kv_cache), _ptr(block_table), max_pages, page_size,
                                _ptr(ctx_len), int(max_ctx), _ptr(out), _ptr(lse), float(scale),
                                int(nsplit), b, lq, h, kv_cache.shape[0], _ptr(ws), ws_bytes,
                                _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_decode_dense")
    return nsplit


def partials_view(ws: torch.Tensor, batch: int, q_len: int, heads: int, nsplit: int):
    """(part_o [T, S, H, 512], part_lse [T, S, H]) views into a workspace."""
    t = batch * q_len
    n_o = t * nsplit * heads * DV
    off = smla_workspace_lse_offset(batch, q_len, heads, nsplit)
    part_o = ws[WS_SYNC_BYTES: WS_SYNC_BYTES + n_o * 4].view(torch.float32).view(t, nsplit, heads, DV)
    part_lse = ws[off: off + t * nsplit * heads * 4].view(torch.float32).view(t, nsplit, heads)
    return part_o, part_lse


def smla_combine(part_o: torch.Tensor, part_lse: torch.Tensor, out: torch.Tensor,
                 lse: torch.Tensor, stream=None) -> None:
    """Combine kernel alone: part_o [T, S, H, 512] fp32, part_lse [T, S, H] fp32."""
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise TypeError("partials must be float32")
    if not (part_o.is_contiguous() and part_lse.is_contiguous()):
        raise ValueError("partials must be contiguous")
    t, s, h = part_lse.shape
    if tuple(part_o.shape) != (t, s, h, DV):
        raise ValueError(f"part_o must be [{t}, {s}, {h}, {DV}], got {tuple(part_o.shape)}")
    rc = _lib_handle().smla_combine(_ptr(part_o), _ptr(part_lse), _ptr(out), _ptr(lse), t, h, s,
                           _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_combine")


def smla_topk_workspace_bytes(batch: int, q_len: int, max_ctx: int) -> int:
    return int(_lib_handle().smla_topk_workspace_bytes(batch, q_len, max_ctx))


def smla_set_topk_min_chunks(min_chunks: int) -> int:
    """Chunk count from which smla_topk spreads a row over several workgroups
    (0 = never); returns the previous value."""
    r = _lib_handle().smla_set_topk_min_chunks(min_chunks)
    if r < 0:
        raise SmlaError(r, "smla_set_topk_min_chunks")
    return r


def smla_topk(scores: torch.Tensor, topk: int, out_pos: torch.Tensor, ctx_len=None, stream=None,
              workspace_t="auto") -> None:
    """Top-k producer: out_pos [B, Lq, topk] int32 = the positions of the topk
    largest of scores [B, Lq, max_ctx] fp32 among positions < ctx_len[b]
    (all when ctx_len is None), ascending, -1 padded (ranking as in
    include/smla.h).  workspace_t: "auto" allocates the multi-workgroup
    form's workspace, None runs one workgroup per row, or a uint8 tensor."""
    if scores.dtype != torch.float32 or not scores.is_contiguous() or scores.dim() != 3:
        raise ValueError("scores must be a contiguous float32 [batch, q_len, max_ctx] tensor")
    b, lq, max_ctx = scores.shape
    if out_pos.dtype != torch.int32 or not out_pos.is_contiguous() or tuple(out_pos.shape) != (b, lq, topk):
        raise ValueError(f"out_pos must be a contiguous int32 [{b}, {lq}, {topk}] tensor")
    if ctx_len is not None and (ctx_len.dtype != torch.int32 or tuple(ctx_len.shape) != (b,)
                                or not ctx_len.is_contiguous()):
        raise ValueError("ctx_len must be a contiguous int32 [batch] tensor")
    ws = workspace_t
    if isinstance(ws, str):
        n = smla_topk_workspace_bytes(b, lq, max_ctx)
        ws = torch.empty(n, dtype=torch.uint8, device=scores.device) if n else None
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = _lib_handle().smla_topk(_ptr(scores), _ptr(ctx_len), b, lq, max_ctx, int(topk), _ptr(out_pos),
                                 _ptr(ws), ws_bytes, _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_topk")
