"""ctypes binding of libsmla.so (include/smla.h).

Argument marshalling only: every function checks the torch tensors it is handed
(device, dtype, shape, contiguity), passes their device pointers and the current
HIP stream to the C entry point of the same name, and raises on a non-zero
status.  All computation happens in the HIP kernels of the library.  If the
library is not built, the first call raises -- there is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsmla.so")

ROW_BYTES = 352
HEAD_DIM = 576
LATENT_DIM = 512

_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "smla_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "nvfp4_pack_rows": ([_P, _P, _I32, _P, _I64, _P], ctypes.c_int),
    "nvfp4_unpack_rows_f16": ([_P, _I64, _P, _I32, _P, _P], ctypes.c_int),
    "sparse_mla_decode": ([_P, _P, _I64, _P, _I32, _I32, _I32, _F32, _P, _P, _I32, _P, _SZ, _P], ctypes.c_int),
    "sparse_mla_decode_noalloc": ([_P, _P, _I64, _P, _I32, _I32, _I32, _F32, _P, _P, _I32, _P], ctypes.c_int),
    "smla_choose_num_splits": ([_I32, _I32, _I32], _I32),
    "smla_decode_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "sparse_mla_combine": ([_P, _P, _I32, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "nvfp4_stage_fp8": ([_P, _I64, _P, _I32, _I32, _P, _P], ctypes.c_int),
    "sparse_mla_decode_fp8rows": ([_P, _P, _P, _I64, _I32, _I32, _I32, _F32, _P, _P, _I32, _P, _SZ, _P], ctypes.c_int),
    "fp8_pack_rows": ([_P, _P, _I32, _P, _I64, _P], ctypes.c_int),
    "sparse_mla_decode_fp8pool": ([_P, _P, _I64, _P, _I32, _I32, _I32, _F32, _P, _P, _I32, _P, _SZ, _P],
                                  ctypes.c_int),
    "sparse_indexer_topk": ([_P, _I64, _P, _P, _I32, _I32, _P, _I32, _P, _SZ, _P], ctypes.c_int),
    "smla_indexer_workspace_bytes": ([_I32, _I64, _I32, _I32], _SZ),
    "smla_group_union": ([_P, _I32, _I32, _I32, _I64, _I32, _P, _P, _P], ctypes.c_int),
    "sparse_mla_decode_grouped": ([_P, _P, _I64, _P, _I32, _I32, _I32, _I32, _F32, _P, _P, _I32, _P, _SZ, _P],
                                  ctypes.c_int),
    "smla_decode_grouped_workspace_bytes": ([_I32, _I32, _I32, _I32, _I32], _SZ),
    "nvfp4_pack_rows_blhnc": ([_P, _P, _I32, _P, _I64, _I32, _I32, _I32, _P], ctypes.c_int),
    "sparse_mla_decode_blhnc": ([_P, _P, _I64, _I32, _I32, _I32, _P, _I32, _I32, _I32, _F32, _P, _P, _I32, _P,
                                 _SZ, _P], ctypes.c_int),
    "blhnc_copy_blocks": ([_P, _I64, _P, _P, _I64, _P, _I32, _I64, _P], ctypes.c_int),
}

EXPORTS = tuple(_SIGS)


class SmlaError(RuntimeError):
    pass


def lib():
    """Load libsmla.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SmlaError(f"{LIB_PATH} is not built; run `python -m sparse_mla_decode_04_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(status, what):
    if status != 0:
        msg = lib().smla_status_string(status).decode()
        raise SmlaError(f"{what} failed: {msg} ({status})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def nvfp4_pack_rows(src, slots, kv_pool):
    """Quantize fp16 rows src[n, 576] into 352-byte rows of kv_pool[N, 352] at slots[n]."""
    n = src.shape[0] if src.dim() == 2 else -1
    p_src = _dev(src, "src", torch.float16, (n, HEAD_DIM))
    p_slots = _dev(slots, "slots", torch.int32, (n,))
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    p_pool = _dev(kv_pool, "kv_pool", torch.uint8)
    _check(lib().nvfp4_pack_rows(p_src, p_slots, n, p_pool, kv_pool.shape[0], _stream()), "nvfp4_pack_rows")


def nvfp4_unpack_rows_f16(kv_pool, rows, out=None):
    """fp16 [n, 576] decode of the cache rows `rows` (int32 [n])."""
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    n = rows.shape[0]
    if out is None:
        out = torch.empty((n, HEAD_DIM), dtype=torch.float16, device=kv_pool.device)
    _check(lib().nvfp4_unpack_rows_f16(_dev(kv_pool, "kv_pool", torch.uint8), kv_pool.shape[0],
                                       _dev(rows, "rows", torch.int32, (n,)), n,
                                       _dev(out, "out", torch.float16, (n, HEAD_DIM)), _stream()),
           "nvfp4_unpack_rows_f16")
    return out


def choose_num_splits(T, H, topk):
    return int(lib().smla_choose_num_splits(T, H, topk))


def decode_workspace_bytes(T, H, topk, num_splits=0):
    return int(lib().smla_decode_workspace_bytes(T, H, topk, num_splits))


def make_workspace(T, H, topk, num_splits=0, device="cuda"):
    """Zero-filled workspace for sparse_mla_decode (uint8 tensor, possibly empty)."""
    nb = decode_workspace_bytes(T, H, topk, num_splits)
    return torch.zeros(max(nb, 16), dtype=torch.uint8, device=device)


def _decode_common(entry, q, rows, pool_rows, indices, softmax_scale, out, lse, num_splits, workspace):
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be fp16 [T, H, 576]")
    T, H, _ = q.shape
    if indices.dim() != 2 or indices.shape[0] != T:
        raise ValueError("indices must be int32 [T, topk]")
    topk = indices.shape[1]
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = make_workspace(T, H, topk, num_splits, q.device)
    p_ws = _dev(workspace, "workspace", torch.uint8)
    p_q = _dev(q, "q", torch.float16)
    p_idx = _dev(indices, "indices", torch.int32)
    tail = (T, H, topk, float(softmax_scale), _dev(out, "out", torch.float16, (T, H, LATENT_DIM)),
            _dev(lse, "lse", torch.float32, (T, H)), int(num_splits), p_ws, workspace.numel(), _stream())
    if entry == "sparse_mla_decode":
        st = lib().sparse_mla_decode(p_q, rows, pool_rows, p_idx, *tail)
    elif entry == "sparse_mla_decode_blhnc":
        nb, layers, layer, B = pool_rows   # the block-major layout
        st = lib().sparse_mla_decode_blhnc(p_q, rows, nb, layers, layer, B, p_idx, *tail)
    elif entry == "sparse_mla_decode_fp8pool":
        st = lib().sparse_mla_decode_fp8pool(p_q, rows, pool_rows, p_idx, *tail)
    else:
        st = lib().sparse_mla_decode_fp8rows(p_q, rows, p_idx, pool_rows, *tail)
    _check(st, entry)
    return out, lse


def sparse_mla_decode(q, kv_pool, indices, softmax_scale, out=None, lse=None, num_splits=0, workspace=None):
    """Sparse MLA decode: returns (out fp16 [T, H, 512], lse fp32 [T, H])."""
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    return _decode_common("sparse_mla_decode", q, _dev(kv_pool, "kv_pool", torch.uint8), kv_pool.shape[0],
                          indices, softmax_scale, out, lse, num_splits, workspace)


def sparse_mla_decode_noalloc(q, kv_pool, indices, softmax_scale, out=None, lse=None, num_splits=0):
    """sparse_mla_decode without a workspace: the library's own scratch holds the split
    partials (SMLA_NOALLOC_SCRATCH_BYTES per GPU; calls overlapping on one GPU race)."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be fp16 [T, H, 576]")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    T, H, _ = q.shape
    topk = indices.shape[1]
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    _check(lib().sparse_mla_decode_noalloc(
        _dev(q, "q", torch.float16, (T, H, HEAD_DIM)), _dev(kv_pool, "kv_pool", torch.uint8),
        ctypes.c_int64(kv_pool.shape[0]), _dev(indices, "indices", torch.int32, (T, topk)), T, H, topk,
        ctypes.c_float(softmax_scale), _dev(out, "out", torch.float16, (T, H, LATENT_DIM)),
        _dev(lse, "lse", torch.float32, (T, H)), int(num_splits), _stream()), "sparse_mla_decode_noalloc")
    return out, lse


def sparse_mla_combine(partial_out, partial_lse, out=None, lse=None):
    """LSE merge of split results: partial_out fp32 [T, S, H, 512], partial_lse fp32 [T, S, H]."""
    if partial_out.dim() != 4 or partial_out.shape[3] != LATENT_DIM:
        raise ValueError("partial_out must be fp32 [T, S, H, 512]")
    T, S, H, _ = partial_out.shape
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=torch.float16, device=partial_out.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=partial_out.device)
    _check(lib().sparse_mla_combine(_dev(partial_out, "partial_out", torch.float32),
                                    _dev(partial_lse, "partial_lse", torch.float32, (T, S, H)), T, S, H,
                                    _dev(out, "out", torch.float16, (T, H, LATENT_DIM)),
                                    _dev(lse, "lse", torch.float32, (T, H)), _stream()),
           "sparse_mla_combine")
    return out, lse


def nvfp4_stage_fp8(kv_pool, indices, staged=None):
    """Staged pass 1: uint8 [T, topk, 576] E4M3 rows of the listed entries (zeros for empties)."""
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    T, topk = indices.shape
    if staged is None:
        staged = torch.empty((T, topk, HEAD_DIM), dtype=torch.uint8, device=kv_pool.device)
    _check(lib().nvfp4_stage_fp8(_dev(kv_pool, "kv_pool", torch.uint8), kv_pool.shape[0],
                                 _dev(indices, "indices", torch.int32), T, topk,
                                 _dev(staged, "staged", torch.uint8, (T, topk, HEAD_DIM)), _stream()),
           "nvfp4_stage_fp8")
    return staged


def sparse_mla_decode_fp8rows(q, staged, indices, pool_rows, softmax_scale, out=None, lse=None,
                              num_splits=0, workspace=None):
    """Staged pass 2: attention over the FP8 rows written by nvfp4_stage_fp8."""
    T, topk = indices.shape
    p_st = _dev(staged, "staged", torch.uint8, (T, topk, HEAD_DIM))
    return _decode_common("sparse_mla_decode_fp8rows", q, p_st, int(pool_rows), indices, softmax_scale,
                          out, lse, num_splits, workspace)


def fp8_pack_rows(src, slots, fp8_pool):
    """Encode fp16 rows src[n, 576] as 576-byte E4M3 rows of fp8_pool[N, 576] at slots[n]."""
    n = src.shape[0] if src.dim() == 2 else -1
    p_src = _dev(src, "src", torch.float16, (n, HEAD_DIM))
    p_slots = _dev(slots, "slots", torch.int32, (n,))
    if fp8_pool.dim() != 2 or fp8_pool.shape[1] != HEAD_DIM:
        raise ValueError("fp8_pool must be uint8 [N, 576]")
    p_pool = _dev(fp8_pool, "fp8_pool", torch.uint8)
    _check(lib().fp8_pack_rows(p_src, p_slots, n, p_pool, fp8_pool.shape[0], _stream()), "fp8_pack_rows")


def sparse_mla_decode_fp8pool(q, fp8_pool, indices, softmax_scale, out=None, lse=None, num_splits=0,
                              workspace=None):
    """Sparse MLA decode over a pool of 576-byte FP8 rows: (out fp16 [T, H, 512], lse fp32 [T, H])."""
    if fp8_pool.dim() != 2 or fp8_pool.shape[1] != HEAD_DIM:
        raise ValueError("fp8_pool must be uint8 [N, 576]")
    return _decode_common("sparse_mla_decode_fp8pool", q, _dev(fp8_pool, "fp8_pool", torch.uint8),
                          fp8_pool.shape[0], indices, softmax_scale, out, lse, num_splits, workspace)


def prepare_decode(q, kv_pool, indices, softmax_scale, out, lse, num_splits=0, workspace=None):
    """Check the arguments of sparse_mla_decode once and return a zero-argument callable
    that enqueues it on the current stream with the marshalled pointers (for loops that
    launch the same shapes many times)."""
    T, H, _ = q.shape
    topk = indices.shape[1]
    if workspace is None:
        workspace = make_workspace(T, H, topk, num_splits, q.device)
    args = (_dev(q, "q", torch.float16, (T, H, HEAD_DIM)), _dev(kv_pool, "kv_pool", torch.uint8),
            ctypes.c_int64(kv_pool.shape[0]), _dev(indices, "indices", torch.int32, (T, topk)),
            T, H, topk, ctypes.c_float(softmax_scale), _dev(out, "out", torch.float16, (T, H, LATENT_DIM)),
            _dev(lse, "lse", torch.float32, (T, H)), int(num_splits), _dev(workspace, "workspace", torch.uint8),
            ctypes.c_size_t(workspace.numel()))
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    fn = lib().sparse_mla_decode
    keep = (q, kv_pool, indices, out, lse, workspace)   # keep the tensors alive

    def call():
        st = fn(*args, _stream())
        if st != 0:
            _check(st, "sparse_mla_decode")
    call.tensors = keep
    return call


def prepare_pack(src, slots, kv_pool):
    """Like prepare_decode, for nvfp4_pack_rows."""
    n = src.shape[0]
    args = (_dev(src, "src", torch.float16, (n, HEAD_DIM)), _dev(slots, "slots", torch.int32, (n,)), n,
            _dev(kv_pool, "kv_pool", torch.uint8), ctypes.c_int64(kv_pool.shape[0]))
    fn = lib().nvfp4_pack_rows
    keep = (src, slots, kv_pool)

    def call():
        st = fn(*args, _stream())
        if st != 0:
            _check(st, "nvfp4_pack_rows")
    call.tensors = keep
    return call


# ---------------------------------------------------------------- sparse indexer ---

def indexer_workspace_bytes(T, S, k, parts=0):
    return int(lib().smla_indexer_workspace_bytes(T, S, k, parts))


def make_indexer_workspace(T, S, k, parts=0, device="cuda"):
    """Zero-filled workspace for sparse_indexer_topk (uint8 tensor), or None when the call
    runs one workgroup per token."""
    nb = indexer_workspace_bytes(T, S, k, parts)
    return torch.zeros(nb, dtype=torch.uint8, device=device) if nb > 0 else None


def sparse_indexer_topk(scores, k, lengths=None, row_offset=None, out=None, parts=0, workspace=None):
    """Top-k selection over scores float32 [T, S] (S a multiple of 4): int32 [T, k] lists of
    row_offset[t] + position, ascending, -1 past a token's length.  parts: workgroups per
    token (0 = the library's choice); a workspace is made when the call needs one and none is
    given."""
    if scores.dim() != 2:
        raise ValueError("scores must be float32 [T, S]")
    T, S = scores.shape
    if out is None:
        out = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    p_len = _dev(lengths, "lengths", torch.int32, (T,)) if lengths is not None else None
    p_off = _dev(row_offset, "row_offset", torch.int32, (T,)) if row_offset is not None else None
    if workspace is None:
        workspace = make_indexer_workspace(T, S, k, parts, scores.device)
    p_ws = _dev(workspace, "workspace", torch.uint8) if workspace is not None else None
    nb = workspace.numel() if workspace is not None else 0
    _check(lib().sparse_indexer_topk(_dev(scores, "scores", torch.float32), S, p_len, p_off, T, k,
                                     _dev(out, "out", torch.int32, (T, k)), int(parts), p_ws, nb, _stream()),
           "sparse_indexer_topk")
    return out


# ---------------------------------------------------------------- grouped decode ---

def group_union(indices, tpg, pool_rows, U, union=None, count=None):
    """Union lists of groups of `tpg` consecutive tokens: (union int32 [T/tpg, U],
    count int32 [T/tpg]); entries are row | members << 27, -1 past the union's size."""
    if indices.dim() != 2:
        raise ValueError("indices must be int32 [T, topk]")
    T, topk = indices.shape
    if T % tpg != 0:
        raise ValueError("T must be a multiple of tpg")
    G = T // tpg
    if union is None:
        union = torch.empty((G, U), dtype=torch.int32, device=indices.device)
    if count is None:
        count = torch.empty((G,), dtype=torch.int32, device=indices.device)
    _check(lib().smla_group_union(_dev(indices, "indices", torch.int32), T, topk, tpg, int(pool_rows), U,
                                  _dev(union, "union", torch.int32, (G, U)), _dev(count, "count", torch.int32, (G,)),
                                  _stream()), "smla_group_union")
    return union, count


def grouped_workspace_bytes(T, H, tpg, U, num_splits=0):
    return int(lib().smla_decode_grouped_workspace_bytes(T, H, tpg, U, num_splits))


def make_grouped_workspace(T, H, tpg, U, num_splits=0, device="cuda"):
    """Zero-filled workspace for sparse_mla_decode_grouped (uint8 tensor)."""
    nb = grouped_workspace_bytes(T, H, tpg, U, num_splits)
    return torch.zeros(max(nb, 16), dtype=torch.uint8, device=device)


def sparse_mla_decode_grouped(q, kv_pool, union, tpg, softmax_scale, out=None, lse=None, num_splits=0,
                              workspace=None):
    """Grouped decode over union lists: q fp16 [T, H, 576], union int32 [T/tpg, U]."""
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be fp16 [T, H, 576]")
    if kv_pool.dim() != 2 or kv_pool.shape[1] != ROW_BYTES:
        raise ValueError("kv_pool must be uint8 [N, 352]")
    T, H, _ = q.shape
    U = union.shape[1]
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=torch.float16, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = make_grouped_workspace(T, H, tpg, U, num_splits, q.device)
    _check(lib().sparse_mla_decode_grouped(
        _dev(q, "q", torch.float16), _dev(kv_pool, "kv_pool", torch.uint8), kv_pool.shape[0],
        _dev(union, "union", torch.int32, (T // tpg, U)), T, H, tpg, U, float(softmax_scale),
        _dev(out, "out", torch.float16, (T, H, LATENT_DIM)), _dev(lse, "lse", torch.float32, (T, H)),
        int(num_splits), _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream()),
        "sparse_mla_decode_grouped")
    return out, lse



def _blhnc_pool(pool):
    if pool.dim() != 4 or pool.shape[3] != ROW_BYTES:
        raise ValueError("pool must be uint8 [blocks, layers, block_rows, 352]")
    return _dev(pool, "pool", torch.uint8), int(pool.shape[0]), int(pool.shape[1]), int(pool.shape[2])


def nvfp4_pack_rows_blhnc(src, slots, pool, layer):
    """Quantize fp16 rows src[n, 576] into rows slots[n] of layer `layer` of a block-major
    pool uint8 [blocks, layers, block_rows, 352]."""
    n = src.shape[0] if src.dim() == 2 else -1
    p_src = _dev(src, "src", torch.float16, (n, HEAD_DIM))
    p_slots = _dev(slots, "slots", torch.int32, (n,))
    p_pool, nb, layers, B = _blhnc_pool(pool)
    _check(lib().nvfp4_pack_rows_blhnc(p_src, p_slots, n, p_pool, nb, layers, int(layer), B, _stream()),
           "nvfp4_pack_rows_blhnc")


def sparse_mla_decode_blhnc(q, pool, layer, indices, softmax_scale, out=None, lse=None, num_splits=0,
                            workspace=None):
    """Sparse MLA decode of layer `layer` of a block-major pool uint8 [blocks, layers,
    block_rows, 352]: returns (out fp16 [T, H, 512], lse fp32 [T, H])."""
    p_pool, nb, layers, B = _blhnc_pool(pool)
    return _decode_common("sparse_mla_decode_blhnc", q, p_pool, (nb, layers, int(layer), B), indices,
                          softmax_scale, out, lse, num_splits, workspace)


def blhnc_copy_blocks(src, dst, src_ids=None, dst_ids=None, n=None):
    """Copy whole segments (the first dimension of src and dst, same segment size): segment
    src_ids[i] of src to segment dst_ids[i] of dst (None = segment i)."""
    if src.dim() < 1 or dst.dim() < 1:
        raise ValueError("src and dst must have a segment dimension")
    seg = src[0].numel() * src.element_size() if src.shape[0] else 0
    dseg = dst[0].numel() * dst.element_size() if dst.shape[0] else 0
    if src.shape[0] and dst.shape[0] and seg != dseg:
        raise ValueError("src and dst segments differ in size")
    seg = seg or dseg
    if n is None:
        n = (src_ids if src_ids is not None else dst_ids if dst_ids is not None else src).shape[0]
    if n == 0:
        return dst
    p_src = _dev(src, "src", src.dtype)
    p_dst = _dev(dst, "dst", dst.dtype)
    p_sid = _dev(src_ids, "src_ids", torch.int32) if src_ids is not None else None
    p_did = _dev(dst_ids, "dst_ids", torch.int32) if dst_ids is not None else None
    for ids, name in ((src_ids, "src_ids"), (dst_ids, "dst_ids")):
        if ids is not None and (ids.dim() != 1 or ids.shape[0] < n):
            raise ValueError(f"{name} must be int32 [n]")
    _check(lib().blhnc_copy_blocks(p_src, src.shape[0], p_sid, p_dst, dst.shape[0], p_did, int(n), seg,
                                   _stream()), "blhnc_copy_blocks")
    return dst
