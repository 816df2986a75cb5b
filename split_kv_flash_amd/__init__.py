"""Split-KV (flash-decoding) decode attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libsplitkv.so`` (C ABI in
``include/splitkv.h``): a split kernel in which one workgroup serves every
query head of a KV group (or of a shared latent) over one contiguous slice of
the context, and a combine kernel that rescales the partials to their common
maximum and sums them. ``attn_decode`` runs the two back to back;
``attn_decode_one_launch`` runs both steps in one launch for separate K and V
(the last workgroup of each group to finish merges). This package is the thin Python side: ``binding``
mirrors the C entry points one to one, and :class:`DecodeCall` fills the
descriptor from torch tensors and owns the workspace. PyTorch is used only for
device memory and streams.
"""

from __future__ import annotations

from typing import Optional

from . import binding
from .binding import (  # noqa: F401
    SK_BF16, SK_F16, SK_F32, SK_KV_CONTIGUOUS, SK_KV_PAGED, SkDesc, SkKernelInfo, SkPlan,
    SplitKVError, attn_decode, attn_decode_combine, attn_decode_combine_project,
    attn_decode_kernel_info,
    attn_decode_last_error, attn_decode_no_alloc, attn_decode_one_launch, attn_decode_plan,
    attn_decode_splitk,
    attn_decode_status_string, attn_decode_workspace_bytes, attn_decode_workspace_init,
    attn_query_tiles, attn_query_tiles_plan, attn_query_tiles_workspace_bytes,
)

__all__ = [
    "DecodeCall", "make_desc", "SkDesc", "SkPlan", "SplitKVError", "attn_decode_plan",
    "attn_decode_workspace_bytes", "attn_decode_splitk", "attn_decode_combine",
    "attn_decode_status_string", "attn_decode_last_error", "attn_decode_kernel_info",
    "attn_decode", "attn_decode_one_launch", "attn_decode_no_alloc", "attn_decode_workspace_init",
    "attn_decode_combine_project", "QueryTileCall", "attn_query_tiles", "attn_query_tiles_plan",
    "attn_query_tiles_workspace_bytes", "decode",
]


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: SK_F32, torch.float16: SK_F16, torch.bfloat16: SK_BF16}
    if t.dtype not in codes:
        raise SplitKVError(binding.SK_ERR_UNSUPPORTED, f"dtype {t.dtype} is not f32/f16/bf16")
    return codes[t.dtype]


def make_desc(q, k, v=None, *, scale: float, block_table=None, page_size: int = 0,
              v_cols: Optional[int] = None, max_seq_len: Optional[int] = None) -> SkDesc:
    """Descriptor for tensors laid out as the C header describes.

    q            [B][Hq][Dk], contiguous
    k, v         contiguous cache [B][capacity][Hkv][D] (any strides with unit
                 last stride), or pools [pages][page_size][Hkv][D] when
                 ``block_table`` ([B][max_pages] int32) is given, or row pools
                 [rows][Hkv][D] with ``block_table`` [B][max_indices] naming
                 the pool row of every position (sparse, index-list decode)
    v = None     shared latent: values are the first ``v_cols`` key columns
    """
    d = SkDesc()
    if q.dim() != 3 or not q.is_contiguous():
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, "q must be a contiguous [B][Hq][Dk] tensor")
    B, Hq, Dk = q.shape
    indexed = block_table is not None and k.dim() == 3
    if not indexed and (k.dim() != 4 or k.stride(3) != 1):
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, "k must be 4-D with unit last stride")
    if indexed and k.stride(2) != 1:
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, "a row pool must have unit last stride")
    d.batch, d.num_q_heads, d.head_dim_qk = B, Hq, Dk
    d.num_kv_heads = k.shape[-2]
    if k.shape[-1] != Dk:
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, "k's last dimension must equal q's")
    d.kv_shared = 1 if v is None else 0
    if v is None:
        if v_cols is None:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "v_cols is required without v")
        d.head_dim_v = int(v_cols)
    else:
        if v.shape != k.shape or v.stride() != k.stride() or v.dtype != k.dtype:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "v must match k's shape, strides and dtype")
        d.head_dim_v = v.shape[-1]
    d.scale = float(scale)
    d.q_dtype = _dtype_code(q)
    d.kv_dtype = _dtype_code(k)
    if indexed:
        d.layout = binding.SK_KV_INDEXED
        d.stride_pos, d.stride_head, d.stride_seq = k.stride(0), k.stride(1), 0
        d.max_pages_per_seq = block_table.shape[1]
        d.num_pages = k.shape[0]
        d.page_size = 1
        d.max_seq_len = int(d.max_pages_per_seq if max_seq_len is None else max_seq_len)
    elif block_table is None:
        d.layout = SK_KV_CONTIGUOUS
        d.max_seq_len = int(k.shape[1] if max_seq_len is None else max_seq_len)
        d.stride_seq, d.stride_pos, d.stride_head = k.stride(0), k.stride(1), k.stride(2)
    else:
        if not k.is_contiguous():
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "paged pools must be contiguous")
        d.layout = SK_KV_PAGED
        d.page_size = int(page_size or k.shape[1])
        if k.shape[1] != d.page_size:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "pool dim 1 must equal page_size")
        d.max_pages_per_seq = block_table.shape[1]
        d.num_pages = k.shape[0]
        d.max_seq_len = int(d.max_pages_per_seq * d.page_size if max_seq_len is None else max_seq_len)
    return d


def _on_gpu(*tensors) -> None:
    """Refuses host tensors up front (the kernels take device addresses only)."""
    for t in tensors:
        if t is not None and not getattr(t, "is_cuda", False):
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "tensor arguments must live on the GPU")


def _stream_handle(stream) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


# Splits per chunk of the one-launch decode's merge tree (kMergeChunk in the
# library), and the counter words it keeps per (sequence, KV head).
MERGE_CHUNK = 16


def merge_counter_words(n_splits: int) -> int:
    return 1 + (n_splits + MERGE_CHUNK - 1) // MERGE_CHUNK


class DecodeCall:
    """One decode-attention call shape: descriptor, plan, workspace, outputs.

    ``host_seq_lens`` gives the lengths on the host (for the plan and for the
    contract check 1 <= L_b <= min(capacity, n_splits*chunk)); ``seq_lens`` is
    the same int32 data on the device. Calls launch on the current torch
    stream unless one is given.
    """

    def __init__(self, q, k, v, seq_lens, host_seq_lens, *, scale: float, block_table=None,
                 page_size: int = 0, v_cols: Optional[int] = None, n_splits: int = 0,
                 cu_count: Optional[int] = None, max_seq_len: Optional[int] = None):
        import torch

        _on_gpu(q, k, v, seq_lens, block_table)
        self.desc = make_desc(q, k, v, scale=scale, block_table=block_table, page_size=page_size,
                              v_cols=v_cols, max_seq_len=max_seq_len)
        lens = [int(x) for x in host_seq_lens]
        if len(lens) != self.desc.batch:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "host_seq_lens has the wrong length")
        if cu_count is None:
            cu_count = torch.cuda.get_device_properties(q.device).multi_processor_count
        self.cu_count = int(cu_count)
        self.plan = attn_decode_plan(self.desc, max(lens), sum(lens), self.cu_count, n_splits)
        limit = min(self.desc.max_seq_len, self.plan.n_splits * self.plan.chunk)
        if min(lens) < 1 or max(lens) > limit:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG,
                               f"sequence lengths must lie in [1, {limit}]")
        self.ws_bytes = attn_decode_workspace_bytes(self.desc, self.plan)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=q.device)
        self.init_workspace()
        self.out = torch.empty(self.desc.batch, self.desc.num_q_heads, self.desc.head_dim_v,
                               dtype=torch.float32, device=q.device)
        self.lse = torch.empty(self.desc.batch, self.desc.num_q_heads, dtype=torch.float32,
                               device=q.device)
        self.q, self.k, self.v, self.seq_lens, self.block_table = q, k, v, seq_lens, block_table

    def splitk(self, stream=None):
        attn_decode_splitk(self.desc, self.plan, self.q, self.k, self.v, self.block_table,
                           self.seq_lens, self.workspace, self.ws_bytes, _stream_handle(stream))

    def combine(self, stream=None, with_lse: bool = True):
        attn_decode_combine(self.desc, self.plan, self.seq_lens, self.workspace, self.ws_bytes,
                            self.out, self.lse if with_lse else None, _stream_handle(stream))

    def __call__(self, stream=None):
        """Two launches: the split kernel, then the combine kernel."""
        self.splitk(stream)
        self.combine(stream)
        return self.out, self.lse

    def init_workspace(self, stream=None):
        """Zero the completion counters that :meth:`decode_one_launch` needs (once
        after the workspace is allocated or overwritten)."""
        attn_decode_workspace_init(self.desc, self.plan, self.workspace, self.ws_bytes,
                                   _stream_handle(stream))

    def decode(self, stream=None, with_lse: bool = True):
        """The whole call through ``attn_decode`` (split kernel, then combine)."""
        attn_decode(self.desc, self.plan, self.q, self.k, self.v, self.block_table, self.seq_lens,
                    self.workspace, self.ws_bytes, self.out, self.lse if with_lse else None,
                    _stream_handle(stream))
        return self.out, self.lse

    def decode_one_launch(self, stream=None, with_lse: bool = True):
        """The whole call in one launch (``attn_decode_one_launch``; a shared
        latent runs as a cooperative launch with a grid barrier before the
        merge)."""
        attn_decode_one_launch(self.desc, self.plan, self.q, self.k, self.v, self.block_table,
                               self.seq_lens, self.workspace, self.ws_bytes, self.out,
                               self.lse if with_lse else None, _stream_handle(stream))
        return self.out, self.lse

    def decode_no_alloc(self, stream=None, with_lse: bool = True):
        """The whole call without this object's workspace
        (``attn_decode_no_alloc``: the library's per-device scratch holds the
        partials)."""
        attn_decode_no_alloc(self.desc, self.plan, self.q, self.k, self.v, self.block_table,
                             self.seq_lens, self.out, self.lse if with_lse else None,
                             _stream_handle(stream))
        return self.out, self.lse

    def combine_project(self, w_proj, out, stream=None, with_lse: bool = True):
        """Combine the partials and apply the per-head projection ``w_proj``
        ([Hq][P][Dv], f32/f16/bf16) into ``out`` ([B][Hq][P] f32)."""
        attn_decode_combine_project(self.desc, self.plan, self.seq_lens, self.workspace,
                                    self.ws_bytes, w_proj, _dtype_code(w_proj), w_proj.shape[1],
                                    out, self.lse if with_lse else None, _stream_handle(stream))
        return out, self.lse

    def counters(self):
        """View of the workspace's completion counters, int32 [B][Hkv][W]: per
        (sequence, KV head) the one-launch merge tree's count of finished
        chunks, then one count per chunk of MERGE_CHUNK splits."""
        import torch

        d, p = self.desc, self.plan
        rows = d.batch * d.num_q_heads * p.n_splits

        def a256(x):
            return (x + 255) // 256 * 256

        off = a256(rows * d.head_dim_v * 4) + 2 * a256(rows * 4)
        w = merge_counter_words(p.n_splits)
        n = d.batch * d.num_kv_heads * w
        return self.workspace[off:off + 4 * n].view(torch.int32).view(d.batch, d.num_kv_heads, w)

    def partials(self):
        """Views of the workspace: acc [B][Hq][S][Dv], m and l [B][Hq][S] (f32)."""
        import torch

        d, p = self.desc, self.plan
        rows = d.batch * d.num_q_heads * p.n_splits

        def a256(x):
            return (x + 255) // 256 * 256

        acc_b = rows * d.head_dim_v * 4
        m_off = a256(acc_b)
        l_off = m_off + a256(rows * 4)
        ws = self.workspace
        acc = ws[:acc_b].view(torch.float32).view(d.batch, d.num_q_heads, p.n_splits, d.head_dim_v)
        m = ws[m_off:m_off + rows * 4].view(torch.float32).view(d.batch, d.num_q_heads, p.n_splits)
        l = ws[l_off:l_off + rows * 4].view(torch.float32).view(d.batch, d.num_q_heads, p.n_splits)
        return acc, m, l


class QueryTileCall:
    """Several query positions per sequence (``attn_query_tiles``): q is
    [B][q_len][Hq][D]; query t of sequence b attends positions
    [0, L_b - q_len + t]. Owns the plan, workspace and outputs
    (out [B][q_len][Hq][D], lse [B][q_len][Hq])."""

    def __init__(self, q, k, v, seq_lens, host_seq_lens, *, scale: float, n_splits: int = 0,
                 cu_count: Optional[int] = None):
        import torch

        _on_gpu(q, k, v, seq_lens)
        if q.dim() != 4 or not q.is_contiguous():
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "q must be a contiguous [B][Q][Hq][D] tensor")
        B, Q, Hq, D = q.shape
        self.q_len = int(Q)
        # The descriptor of one query position: [B][Hq][D].
        self.desc = make_desc(q[:, 0].contiguous(), k, v, scale=scale)
        lens = [int(x) for x in host_seq_lens]
        if len(lens) != B:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, "host_seq_lens has the wrong length")
        if cu_count is None:
            cu_count = torch.cuda.get_device_properties(q.device).multi_processor_count
        self.plan = attn_query_tiles_plan(self.desc, self.q_len, max(lens), sum(lens),
                                          int(cu_count), n_splits)
        limit = min(self.desc.max_seq_len, self.plan.n_splits * self.plan.chunk)
        if min(lens) < 1 or max(lens) > limit:
            raise SplitKVError(binding.SK_ERR_INVALID_ARG, f"sequence lengths must lie in [1, {limit}]")
        self.ws_bytes = attn_query_tiles_workspace_bytes(self.desc, self.plan, self.q_len)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=q.device)
        self.out = torch.empty(B, Q, Hq, D, dtype=torch.float32, device=q.device)
        self.lse = torch.empty(B, Q, Hq, dtype=torch.float32, device=q.device)
        self.q, self.k, self.v, self.seq_lens = q, k, v, seq_lens

    def __call__(self, stream=None, with_lse: bool = True):
        attn_query_tiles(self.desc, self.plan, self.q_len, self.q, self.k, self.v, self.seq_lens,
                         self.workspace, self.ws_bytes, self.out, self.lse if with_lse else None,
                         _stream_handle(stream))
        return self.out, self.lse


def decode(q, k, v=None, *, seq_lens, scale: float, n_splits: int = 0, block_table=None,
           page_size: int = 0, v_cols: Optional[int] = None, host_seq_lens=None, out=None,
           lse=None, workspace=None, stream=None):
    """One decode-attention call in a single function: plan, workspace and
    ``attn_decode`` (split kernel, then combine) on the current torch stream.

    ``seq_lens`` is the int32 [B] device tensor the kernels read. The plan
    needs the longest and the total length on the host: pass them as
    ``host_seq_lens`` (any int sequence), or they are copied from
    ``seq_lens``, which synchronises the stream. ``out`` ([B][Hq][Dv] f32),
    ``lse`` ([B][Hq] f32) and ``workspace`` (uint8, at least
    ``attn_decode_workspace_bytes``) are allocated when not given; a given
    workspace must have had ``attn_decode_workspace_init`` only if it is also
    used with ``attn_decode_one_launch``. Returns (out, lse); lse is None
    unless requested with ``lse=True`` or given as a tensor."""
    import torch

    _on_gpu(q, k, v, seq_lens, block_table, out, workspace)
    if isinstance(lse, torch.Tensor):
        _on_gpu(lse)
    desc = make_desc(q, k, v, scale=scale, block_table=block_table, page_size=page_size,
                     v_cols=v_cols)
    lens = [int(x) for x in (seq_lens.tolist() if host_seq_lens is None else host_seq_lens)]
    if len(lens) != desc.batch:
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, "seq_lens has the wrong length")
    cu = torch.cuda.get_device_properties(q.device).multi_processor_count
    plan = attn_decode_plan(desc, max(lens), sum(lens), cu, n_splits)
    limit = min(desc.max_seq_len, plan.n_splits * plan.chunk)
    if min(lens) < 1 or max(lens) > limit:
        raise SplitKVError(binding.SK_ERR_INVALID_ARG, f"sequence lengths must lie in [1, {limit}]")
    ws_bytes = attn_decode_workspace_bytes(desc, plan)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < ws_bytes:
        raise SplitKVError(binding.SK_ERR_WORKSPACE_TOO_SMALL,
                           f"workspace holds {workspace.numel() * workspace.element_size()} "
                           f"bytes, the plan needs {ws_bytes}")
    if out is None:
        out = torch.empty(desc.batch, desc.num_q_heads, desc.head_dim_v, dtype=torch.float32,
                          device=q.device)
    if lse is True:
        lse = torch.empty(desc.batch, desc.num_q_heads, dtype=torch.float32, device=q.device)
    elif lse is False:
        lse = None
    attn_decode(desc, plan, q, k, v, block_table, seq_lens, workspace,
                workspace.numel() * workspace.element_size(), out, lse, _stream_handle(stream))
    return out, lse
