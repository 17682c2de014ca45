"""Python binding of libsmla.so -- sparse MLA decode with split-K over the
top-k list on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/smla.h).  torch supplies device memory and
the stream; there is no CPU fallback.  The library is loaded on first use
(so that the package's build module can run before it exists): any call
without the built library raises ImportError.

Functions carry the C names: smla_plan_nsplit, smla_plan_nsplit_cus,
smla_workspace_bytes, smla_workspace_lse_offset, smla_decode, smla_decode_fused,
smla_fused_in_launch, smla_decode_paged, smla_decode_dense, smla_plan_nsplit_dense,
smla_split, smla_combine, smla_topk, smla_topk_workspace_bytes, smla_decode_noalloc,
smla_status_str.

Every tensor argument is checked before the library is called: dtype,
contiguity, shape, and that it lives on the same GPU as q (the C ABI takes
raw pointers and cannot check any of that itself).
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
MAX_HEADS = 4096
FUSED_SYNC_BYTES = 16384  # SMLA_FUSED_SYNC_BYTES
NOALLOC_SCRATCH_BYTES = 64 << 20  # SMLA_NOALLOC_SCRATCH_BYTES
DEFAULT_MERGE_POLLS = 2048
TOPK_AUTO, TOPK_ROWS, TOPK_CHUNKS, TOPK_SAMPLED = 0, 1, 2, 3  # smla_topk_form

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
    call = [vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i64, vp, sz, vp]
    lib.smla_decode.argtypes = call
    lib.smla_decode.restype = i32
    lib.smla_decode_fused.argtypes = call[:-1] + [vp, sz, i32, vp]
    lib.smla_decode_noalloc.argtypes = call[:-3] + [vp]
    lib.smla_decode_noalloc.restype = i32
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
    lib.smla_topk.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, sz, i32, vp]
    lib.smla_topk.restype = i32
    lib.smla_topk_workspace_bytes.argtypes = [i32, i32, i32]
    lib.smla_topk_workspace_bytes.restype = sz
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


def _check_one(name, t, dtype, shape=None):
    """t must be a contiguous `dtype` tensor, of `shape` when one is given;
    None passes (the caller decides whether the argument is optional)."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")


def _check_devices(device, **tensors):
    """Every given tensor on `device`, a GPU (checked after the shapes, so a
    shape error is reported the same way with or without a GPU)."""
    if device.type != "cuda":
        raise ValueError(f"the tensors must be on a GPU, got {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_tensors(q, kv_cache, topk_idx, out, lse, out_required=True, **more):
    """q [b, lq, h, 576] bf16; kv_cache [rows, 576] bf16; topk_idx int32;
    out [b, lq, h, 512] bf16 and lse [b, lq, h] fp32; all of them, and the
    tensors in `more` (already shape-checked by the caller), on q's GPU."""
    _check_one("q", q, torch.bfloat16)
    if q is None or q.dim() != 4 or q.shape[-1] != ROW:
        raise ValueError(f"q must be [batch, q_len, heads, {ROW}], got "
                         f"{None if q is None else tuple(q.shape)}")
    if q.shape[2] < 1 or q.shape[2] > MAX_HEADS:
        raise ValueError(f"q must have 1 .. {MAX_HEADS} heads, got {q.shape[2]}")
    b, lq, h, _ = q.shape
    _check_one("kv_cache", kv_cache, torch.bfloat16)
    if kv_cache is None or kv_cache.dim() != 2 or kv_cache.shape[1] != ROW:
        raise ValueError(f"kv_cache must be [rows, {ROW}], got "
                         f"{None if kv_cache is None else tuple(kv_cache.shape)}")
    _check_one("topk_idx", topk_idx, torch.int32)
    if topk_idx is not None and (topk_idx.dim() != 3 or tuple(topk_idx.shape[:2]) != (b, lq)):
        raise ValueError(f"topk_idx must be [{b}, {lq}, topk], got {tuple(topk_idx.shape)}")
    if out_required and (out is None or lse is None):
        raise ValueError("out and lse are required")
    _check_one("out", out, torch.bfloat16, (b, lq, h, DV))
    _check_one("lse", lse, torch.float32, (b, lq, h))
    _check_devices(q.device, kv_cache=kv_cache, topk_idx=topk_idx, out=out, lse=lse, **more)


def _check_workspace(ws, device):
    if ws is None:
        return 0
    if not isinstance(ws, torch.Tensor) or ws.device != device:
        raise ValueError(f"the workspace must be a tensor on {device}")
    if not ws.is_contiguous():
        raise ValueError("the workspace must be contiguous")
    return ws.numel() * ws.element_size()


def workspace(batch: int, q_len: int, heads: int, nsplit: int, device) -> torch.Tensor | None:
    """A workspace tensor of the size the call needs (None when nsplit <= 1).
    Its content on entry does not matter."""
    n = smla_workspace_bytes(batch, q_len, heads, nsplit)
    if not n:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def fused_sync(device) -> torch.Tensor:
    """Zeroed synchronisation words for smla_decode_fused (every call leaves
    them zero, so one buffer serves any sequence of calls on one stream)."""
    return torch.zeros(FUSED_SYNC_BYTES, dtype=torch.uint8, device=device)


def _call(fn, name, q, kv_cache, topk_idx, out, lse, scale, nsplit, ws, stream, extra=(),
          out_required=True):
    _check_tensors(q, kv_cache, topk_idx, out, lse, out_required)
    if topk_idx is None:
        raise ValueError("topk_idx is required")
    b, lq, h, k = _shape(q, topk_idx)
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit(b, lq, h, k)
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = _check_workspace(ws, q.device)
    rc = fn(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(out), _ptr(lse), float(scale),
            int(nsplit), b, lq, h, k, kv_cache.shape[0], _ptr(ws), ws_bytes, *extra,
            _stream(stream))
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


def smla_decode_noalloc(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int = 0,
                        stream=None) -> int:
    """smla_decode with its partials in the library's static per-device
    scratch array (no workspace, nothing allocated: see include/smla.h).
    Returns the NSPLIT used."""
    _check_tensors(q, kv_cache, topk_idx, out, lse)
    if topk_idx is None:
        raise ValueError("topk_idx is required")
    b, lq, h, k = _shape(q, topk_idx)
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit(b, lq, h, k)
    rc = _lib_handle().smla_decode_noalloc(_ptr(q), _ptr(kv_cache), _ptr(topk_idx), _ptr(out), _ptr(lse),
                                           float(scale), int(nsplit), b, lq, h, k, kv_cache.shape[0],
                                           _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_decode_noalloc")
    return nsplit


def smla_decode_fused(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int = 0,
                      workspace_t=None, sync=None, merge_polls: int = DEFAULT_MERGE_POLLS,
                      stream=None) -> int:
    """smla_decode with the merge inside the split launch when the shape
    allows it (smla_fused_in_launch), else exactly smla_decode.  sync: the
    zeroed synchronisation words (fused_sync(); allocated when None), which
    every call leaves zero.  Returns the NSPLIT used."""
    _check_one("sync", sync, torch.uint8)
    _check_tensors(q, kv_cache, topk_idx, out, lse, sync=sync)
    if sync is None:
        sync = fused_sync(q.device)
    extra = (_ptr(sync), sync.numel(), int(merge_polls))
    return _call(_lib_handle().smla_decode_fused, "smla_decode_fused", q, kv_cache, topk_idx, out, lse,
                 scale, nsplit, workspace_t, stream, extra)[0]


def smla_split(q, kv_cache, topk_idx, out, lse, scale: float, nsplit: int,
               workspace_t=None, stream=None):
    """Split kernel alone.  Returns (nsplit, workspace) -- the partials live in
    the workspace (see partials_view) when NSPLIT > 1."""
    return _call(_lib_handle().smla_split, "smla_split", q, kv_cache, topk_idx, out, lse, scale, nsplit,
                 workspace_t, stream, out_required=False)


def _check_table(block_table, what):
    if block_table is None:
        return 0
    _check_one(f"{what}: block_table", block_table, torch.int32)
    if block_table.dim() != 2:
        raise ValueError(f"{what}: block_table must be a contiguous int32 [batch, max_pages] tensor")
    return block_table.shape[1]


def smla_decode_paged(q, kv_cache, block_table, page_size: int, topk_pos, out, lse, scale: float,
                      nsplit: int = 0, workspace_t=None, stream=None) -> int:
    """smla_decode with topk_pos [B, Lq, K] holding positions in each
    sequence, mapped to cache rows through block_table [B, max_pages] inside
    the kernel.  Returns the NSPLIT used."""
    if topk_pos is None:
        raise ValueError("smla_decode_paged: topk_pos is required")
    max_pages = _check_table(block_table, "smla_decode_paged")
    if block_table is None or (isinstance(q, torch.Tensor) and block_table.shape[0] != q.shape[0]):
        raise ValueError("smla_decode_paged: block_table must be [batch, max_pages]")
    _check_tensors(q, kv_cache, topk_pos, out, lse, block_table=block_table)
    b, lq, h, k = _shape(q, topk_pos)
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit(b, lq, h, k)
    ws = workspace_t
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = _check_workspace(ws, q.device)
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
    if ctx_len is None:
        raise ValueError("smla_decode_dense: ctx_len is required")
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be [batch, q_len, heads, 576]")
    b = q.shape[0]
    _check_one("smla_decode_dense: ctx_len", ctx_len, torch.int32, (b,))
    max_pages = _check_table(block_table, "smla_decode_dense")
    if block_table is not None and block_table.shape[0] != b:
        raise ValueError("smla_decode_dense: block_table must be [batch, max_pages]")
    _check_tensors(q, kv_cache, None, out, lse, ctx_len=ctx_len, block_table=block_table)
    b, lq, h, _ = q.shape
    if nsplit == 0 and b * lq > 0:
        nsplit = smla_plan_nsplit_dense(b, lq, h, max_ctx)
    ws = workspace_t
    if ws is None and nsplit > 1:
        ws = workspace(b, lq, h, nsplit, q.device)
    ws_bytes = _check_workspace(ws, q.device)
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
    part_o = ws[: n_o * 4].view(torch.float32).view(t, nsplit, heads, DV)
    part_lse = ws[off: off + t * nsplit * heads * 4].view(torch.float32).view(t, nsplit, heads)
    return part_o, part_lse


def smla_combine(part_o: torch.Tensor, part_lse: torch.Tensor, out: torch.Tensor,
                 lse: torch.Tensor, stream=None) -> None:
    """Combine kernel alone: part_o [T, S, H, 512] fp32, part_lse [T, S, H]
    fp32 into out [T, H, 512] bf16 and lse [T, H] fp32, all on one GPU."""
    _check_one("part_lse", part_lse, torch.float32)
    if part_lse is None or part_lse.dim() != 3:
        raise ValueError("part_lse must be a [tokens, nsplit, heads] tensor")
    t, s, h = part_lse.shape
    for name, x, dt, shp in (("part_o", part_o, torch.float32, (t, s, h, DV)),
                             ("out", out, torch.bfloat16, (t, h, DV)),
                             ("lse", lse, torch.float32, (t, h))):
        if x is None:
            raise ValueError(f"{name} is required")
        if name != "part_o" and x.dim() > len(shp):
            # leading dims [batch, q_len, ...] whose product is the token count
            lead = x.shape[: x.dim() - len(shp) + 1]
            n = 1
            for d in lead:
                n *= d
            if n == t:
                shp = tuple(lead) + shp[1:]
        _check_one(name, x, dt, shp)
    _check_devices(part_lse.device, part_o=part_o, out=out, lse=lse)
    rc = _lib_handle().smla_combine(_ptr(part_o), _ptr(part_lse), _ptr(out), _ptr(lse), t, h, s,
                           _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_combine")


def smla_topk_workspace_bytes(batch: int, q_len: int, max_ctx: int) -> int:
    return int(_lib_handle().smla_topk_workspace_bytes(batch, q_len, max_ctx))


def smla_topk(scores: torch.Tensor, topk: int, out_pos: torch.Tensor, ctx_len=None, stream=None,
              workspace_t="auto", form: int = TOPK_AUTO) -> None:
    """Top-k producer: out_pos [B, Lq, topk] int32 = the positions of the topk
    largest of scores [B, Lq, max_ctx] fp32 among positions < ctx_len[b]
    (all when ctx_len is None), ascending, -1 padded (ranking as in
    include/smla.h).  workspace_t: "auto" allocates the multi-workgroup
    form's workspace, None runs one workgroup per row, or a uint8 tensor.
    form: TOPK_AUTO, TOPK_ROWS, TOPK_CHUNKS or TOPK_SAMPLED (the work split)."""
    _check_one("scores", scores, torch.float32)
    if scores is None or scores.dim() != 3:
        raise ValueError("scores must be a float32 [batch, q_len, max_ctx] tensor")
    dev = scores.device
    b, lq, max_ctx = scores.shape
    if out_pos is None:
        raise ValueError("out_pos is required")
    _check_one("out_pos", out_pos, torch.int32, (b, lq, topk))
    _check_one("ctx_len", ctx_len, torch.int32, (b,))
    _check_devices(dev, out_pos=out_pos, ctx_len=ctx_len)
    ws = workspace_t
    if isinstance(ws, str):
        n = smla_topk_workspace_bytes(b, lq, max_ctx)
        ws = torch.empty(n, dtype=torch.uint8, device=dev) if n else None
    ws_bytes = _check_workspace(ws, dev)
    rc = _lib_handle().smla_topk(_ptr(scores), _ptr(ctx_len), b, lq, max_ctx, int(topk), _ptr(out_pos),
                                 _ptr(ws), ws_bytes, int(form), _stream(stream))
    if rc != 0:
        raise SmlaError(rc, "smla_topk")
