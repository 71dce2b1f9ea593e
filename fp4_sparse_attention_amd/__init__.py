"""Python binding of libcsa2 (CSA2 FP4 sparse-attention decode on MI355X / gfx950).

Argument marshalling only: every function below takes torch tensors that
already live on the GPU, checks their dtype/shape/contiguity, passes raw device
pointers, sizes and torch's current HIP stream to the C ABI declared in
include/csa2.h, and raises Csa2Error on a non-zero status.  All arithmetic runs
in the library's HIP kernels; there is no fallback.  The library is loaded from
this package directory; build it first with
``python -m fp4_sparse_attention_amd.build``.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa2.so")

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_size_t = ctypes.c_size_t

_SIGS = {
    "csa2_abi_version": (_i32, []),
    "csa2_status_str": (ctypes.c_char_p, [_i32]),
    "csa2_fp4_pack": (_i32, [_c_void_p, _i64, _i32, _i64, _c_void_p, _i64, _c_void_p, _i64, _c_void_p]),
    "csa2_fp4_unpack": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _c_void_p, _c_void_p]),
    "csa2_index_full": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "csa2_index_full_fp8": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p]),
    "csa2_index_reindex": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _i32, _c_void_p,
                                  _c_void_p]),
    "csa2_topk_workspace_size": (_size_t, [_i32, _i64, _i32]),
    "csa2_topk": (_i32, [_c_void_p, _i32, _i64, _i64, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t,
                         _c_void_p]),
    "csa2_topk_pool_workspace_size": (_size_t, [_i32, _i64, _i32]),
    "csa2_topk_pool": (_i32, [_c_void_p, _i32, _i64, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                              _c_void_p, _size_t, _c_void_p]),
    "csa2_index_full_pool_workspace_size": (_size_t, [_i32, _i64, _i32]),
    "csa2_index_full_pool_streams": (_i32, [_i32, _i64]),
    "csa2_index_full_pool_batch_workspace_size": (_size_t, [_i32, _i64, _i32]),
    "csa2_index_full_pool": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _c_void_p, _i32,
                                    _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p, _c_void_p,
                                    _c_void_p]),
    "csa2_sparse_decode_workspace_size": (_size_t, [_i32, _i32, _i32]),
    "csa2_sparse_decode": (_i32, [_c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i64, _c_void_p, _c_void_p,
                                  _i32, _f32, _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p]),
    "csa2_swa_merge_workspace_size": (_size_t, [_i32, _i32]),
    "csa2_sparse_swa_decode_workspace_size": (_size_t, [_i32, _i32, _i32]),
    "csa2_sparse_swa_decode": (_i32, [_c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i64, _c_void_p, _c_void_p,
                                      _i32, _c_void_p, _i32, _c_void_p, _c_void_p, _f32, _c_void_p, _c_void_p,
                                      _c_void_p, _size_t, _c_void_p]),
    "csa2_sparse_swa_decode_layers_workspace_size": (_size_t, [_i32, _i32, _i32, _i32]),
    "csa2_sparse_swa_decode_layers": (_i32, [_i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i64, _c_void_p,
                                             _c_void_p, _c_void_p, _i32, _c_void_p, _i32, _c_void_p, _c_void_p, _f32,
                                             _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p]),
    "csa2_sparse_swa_decode_layers_noalloc": (_i32, [_i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i64,
                                                     _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p, _i32,
                                                     _c_void_p, _c_void_p, _f32, _c_void_p, _c_void_p, _c_void_p]),
    "csa2_swa_merge": (_i32, [_c_void_p, _i32, _i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _f32,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size_t, _c_void_p]),
    # paged global KV
    "csa2_fp4_pack_rows": (_i32, [_c_void_p, _i64, _i32, _i64, _c_void_p, _c_void_p, _i64, _c_void_p, _i64,
                                  _c_void_p]),
    "csa2_index_full_paged": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _c_void_p, _i64,
                                     _i32, _c_void_p, _c_void_p]),
    "csa2_index_reindex_paged": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _i64, _i32,
                                        _c_void_p, _i32, _c_void_p, _c_void_p]),
    "csa2_index_full_pool_paged_workspace_size": (_size_t, [_i32, _i64, _i32]),
    "csa2_index_full_pool_paged": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i64, _c_void_p, _c_void_p, _c_void_p,
                                          _i64, _i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _c_void_p,
                                          _c_void_p, _size_t, _c_void_p]),
    "csa2_decode_append": (_i32, [_i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "csa2_absorb_q": (_i32, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "csa2_unabsorb_o": (_i32, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "csa2_sparse_swa_decode_layers_paged": (_i32, [_i32, _c_void_p, _i32, _i32, _c_void_p, _c_void_p, _i32, _i64,
                                                   _c_void_p, _c_void_p, _i64, _i32, _c_void_p, _c_void_p, _i32,
                                                   _c_void_p, _i32, _c_void_p, _c_void_p, _f32, _c_void_p, _c_void_p,
                                                   _c_void_p, _size_t, _c_void_p]),
}

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().csa2_status_str(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")


def lib():
    """The loaded libcsa2 (ctypes.CDLL).  Raises if the library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libcsa2.so not found at {LIB_PATH}; run `python -m fp4_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise Csa2Error(fn, status)


def _need(t, dtype, name, ndim=None):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a GPU tensor")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got {tuple(t.shape)}")


def _dense(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def csa2_abi_version():
    return lib().csa2_abi_version()


def csa2_fp4_pack(x, codes, scales, stream=None):
    """x bf16 [n, C] (rows may be strided) -> codes uint8 [n, C/2], scales uint8 [n, C/16].
    codes / scales may be row-strided views (e.g. one row per sequence of a cache)."""
    _need(x, torch.bfloat16, "x", 2)
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    n, C = x.shape
    if codes.shape != (n, C // 2) or scales.shape != (n, C // 16):
        raise ValueError("codes/scales shape mismatch")
    for t, nm in ((x, "x"), (codes, "codes"), (scales, "scales")):
        if t.stride(1) != 1:
            raise ValueError(f"{nm}: channels must be contiguous")
    st = lib().csa2_fp4_pack(_p(x), n, C, x.stride(0), _p(codes), codes.stride(0), _p(scales), scales.stride(0),
                             _stream(stream))
    _check("csa2_fp4_pack", st)


def csa2_fp4_unpack(codes, scales, x, stream=None):
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    _need(x, torch.bfloat16, "x", 2)
    for t, nm in ((codes, "codes"), (scales, "scales"), (x, "x")):
        _dense(t, nm)
    n, C = x.shape
    if codes.shape != (n, C // 2) or scales.shape != (n, C // 16):
        raise ValueError("codes/scales shape mismatch")
    _check("csa2_fp4_unpack", lib().csa2_fp4_unpack(_p(codes), _p(scales), n, C, _p(x), _stream(stream)))


def _index_full_args(q_idx, k_idx, scores, row_seq, row_limit):
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_idx, torch.uint8, "k_idx", 3)
    _need(scores, torch.float32, "scores", 2)
    for t, nm in ((q_idx, "q_idx"), (k_idx, "k_idx"), (scores, "scores")):
        _dense(t, nm)
    R = q_idx.shape[0]
    B, T, D = k_idx.shape
    if D != 64 or q_idx.shape[1] != 64 or scores.shape != (R, T):
        raise ValueError("index shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    if row_limit is not None:
        _need(row_limit, torch.int64, "row_limit", 1)
    return R, B, T


def csa2_index_full(q_idx, k_idx, scores, row_seq=None, row_limit=None, stream=None):
    """q_idx uint8 [R, 64]; k_idx uint8 [B, T, 64]; scores fp32 [R, T] (written)."""
    R, B, T = _index_full_args(q_idx, k_idx, scores, row_seq, row_limit)
    st = lib().csa2_index_full(_p(q_idx), _p(k_idx), R, B, T, _p(row_seq), _p(row_limit), _p(scores), _stream(stream))
    _check("csa2_index_full", st)


def csa2_index_full_fp8(q_idx, k_idx, scores, row_seq=None, row_limit=None, stream=None):
    """csa2_index_full's scores through the FP8 matrix instruction (approximate; see the header)."""
    R, B, T = _index_full_args(q_idx, k_idx, scores, row_seq, row_limit)
    st = lib().csa2_index_full_fp8(_p(q_idx), _p(k_idx), R, B, T, _p(row_seq), _p(row_limit), _p(scores),
                                   _stream(stream))
    _check("csa2_index_full_fp8", st)


def csa2_index_reindex(q_idx, k_idx, pool, scores, row_seq=None, stream=None):
    """q_idx uint8 [R, 64]; k_idx uint8 [B, T, 64]; pool int32 [R, P]; scores fp32 [R, P]."""
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_idx, torch.uint8, "k_idx", 3)
    _need(pool, torch.int32, "pool", 2)
    _need(scores, torch.float32, "scores", 2)
    for t, nm in ((q_idx, "q_idx"), (k_idx, "k_idx"), (pool, "pool"), (scores, "scores")):
        _dense(t, nm)
    R, P = pool.shape
    B, T, _ = k_idx.shape
    if scores.shape != (R, P) or q_idx.shape != (R, 64):
        raise ValueError("reindex shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    st = lib().csa2_index_reindex(_p(q_idx), _p(k_idx), R, B, T, _p(row_seq), _p(pool), P, _p(scores),
                                  _stream(stream))
    _check("csa2_index_reindex", st)


def csa2_topk_workspace_size(R, N, k):
    return int(lib().csa2_topk_workspace_size(R, N, k))


def csa2_topk(scores, k, idx_out, score_out=None, index_map=None, workspace=None, stream=None):
    """scores fp32 [R, N] (row stride may exceed N); idx_out int32 [R, k]; score_out fp32 [R, k] or None;
    index_map int32 [R, N] or None; workspace uint8 tensor (allocated here if None)."""
    _need(scores, torch.float32, "scores", 2)
    _need(idx_out, torch.int32, "idx_out", 2)
    if scores.stride(1) != 1:
        raise ValueError("scores: columns must be contiguous")
    R, N = scores.shape
    if idx_out.shape != (R, k):
        raise ValueError("idx_out shape")
    _dense(idx_out, "idx_out")
    if score_out is not None:
        _need(score_out, torch.float32, "score_out", 2)
        _dense(score_out, "score_out")
    if index_map is not None:
        _need(index_map, torch.int32, "index_map", 2)
        _dense(index_map, "index_map")
    need = csa2_topk_workspace_size(R, N, k)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    st = lib().csa2_topk(_p(scores), R, N, scores.stride(0), k, _p(index_map), _p(idx_out), _p(score_out),
                         _p(workspace), workspace.numel(), _stream(stream))
    _check("csa2_topk", st)


def csa2_topk_pool_workspace_size(R, N, k_pool):
    return int(lib().csa2_topk_pool_workspace_size(R, N, k_pool))


def csa2_topk_pool(scores, k_pool, k_top, pool_idx, top_idx, pool_scores=None, index_map=None, workspace=None,
                   stream=None):
    """The k_pool and the k_top <= k_pool highest scores of each row in one selection.
    scores fp32 [R, N]; pool_idx int32 [R, k_pool]; top_idx int32 [R, k_top];
    pool_scores fp32 [R, k_pool] or None; index_map int32 [R, N] or None."""
    _need(scores, torch.float32, "scores", 2)
    _need(pool_idx, torch.int32, "pool_idx", 2)
    _need(top_idx, torch.int32, "top_idx", 2)
    if scores.stride(1) != 1:
        raise ValueError("scores: columns must be contiguous")
    R, N = scores.shape
    if pool_idx.shape != (R, k_pool) or top_idx.shape != (R, k_top):
        raise ValueError("pool_idx / top_idx shape")
    _dense(pool_idx, "pool_idx")
    _dense(top_idx, "top_idx")
    if pool_scores is not None:
        _need(pool_scores, torch.float32, "pool_scores", 2)
        if pool_scores.shape != (R, k_pool):
            raise ValueError("pool_scores shape")
        _dense(pool_scores, "pool_scores")
    if index_map is not None:
        _need(index_map, torch.int32, "index_map", 2)
        _dense(index_map, "index_map")
    need = csa2_topk_pool_workspace_size(R, N, k_pool)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=scores.device)
    st = lib().csa2_topk_pool(_p(scores), R, N, scores.stride(0), k_pool, k_top, _p(index_map), _p(pool_idx),
                              _p(pool_scores), _p(top_idx), _p(workspace), workspace.numel(), _stream(stream))
    _check("csa2_topk_pool", st)


def csa2_sparse_decode_workspace_size(R, H, K):
    return int(lib().csa2_sparse_decode_workspace_size(R, H, K))


def csa2_sparse_decode(q_lat, codes, scales, idx, softmax_scale, o, lse, row_seq=None, workspace=None,
                       stream=None):
    """q_lat bf16 [R, H, 512]; codes uint8 [B, T, 256]; scales uint8 [B, T, 32]; idx int32 [R, K];
    o fp32 [R, H, 512]; lse fp32 [R, H]."""
    _need(q_lat, torch.bfloat16, "q_lat", 3)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _need(idx, torch.int32, "idx", 2)
    _need(o, torch.float32, "o", 3)
    _need(lse, torch.float32, "lse", 2)
    for t, nm in ((q_lat, "q_lat"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (o, "o"), (lse, "lse")):
        _dense(t, nm)
    R, H, C = q_lat.shape
    B, T, cb = codes.shape
    K = idx.shape[1]
    if C != 512 or cb != 256 or scales.shape != (B, T, 32) or o.shape != (R, H, 512) or lse.shape != (R, H):
        raise ValueError("sparse_decode shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    need = csa2_sparse_decode_workspace_size(R, H, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    st = lib().csa2_sparse_decode(_p(q_lat), R, H, _p(codes), _p(scales), B, T, _p(row_seq), _p(idx), K,
                                  float(softmax_scale), _p(o), _p(lse), _p(workspace), workspace.numel(),
                                  _stream(stream))
    _check("csa2_sparse_decode", st)


def csa2_swa_merge_workspace_size(R, H):
    return int(lib().csa2_swa_merge_workspace_size(R, H))


def csa2_swa_merge(q_lat, swa, swa_start, swa_len, softmax_scale, o_out, lse_out=None, o_sparse=None,
                   lse_sparse=None, row_seq=None, workspace=None, stream=None):
    """q_lat bf16 [R, H, 512]; swa bf16 [B, S, 512]; swa_start / swa_len int32 [R];
    o_sparse / lse_sparse: the sparse result or None; o_out fp32 [R, H, 512]; lse_out fp32 [R, H] or None."""
    _need(q_lat, torch.bfloat16, "q_lat", 3)
    _need(swa, torch.bfloat16, "swa", 3)
    _need(swa_start, torch.int32, "swa_start", 1)
    _need(swa_len, torch.int32, "swa_len", 1)
    _need(o_out, torch.float32, "o_out", 3)
    for t, nm in ((q_lat, "q_lat"), (swa, "swa"), (swa_start, "swa_start"), (swa_len, "swa_len"),
                  (o_out, "o_out")):
        _dense(t, nm)
    R, H, _ = q_lat.shape
    B, S, C = swa.shape
    if C != 512 or o_out.shape != (R, H, 512) or swa_start.shape != (R,) or swa_len.shape != (R,):
        raise ValueError("swa_merge shapes")
    for t, nm, dt in ((o_sparse, "o_sparse", torch.float32), (lse_sparse, "lse_sparse", torch.float32),
                      (lse_out, "lse_out", torch.float32)):
        if t is not None:
            _need(t, dt, nm)
            _dense(t, nm)
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    need = csa2_swa_merge_workspace_size(R, H)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    st = lib().csa2_swa_merge(_p(q_lat), R, H, _p(swa), B, S, _p(row_seq), _p(swa_start), _p(swa_len),
                              float(softmax_scale), _p(o_sparse), _p(lse_sparse), _p(o_out), _p(lse_out),
                              _p(workspace), workspace.numel(), _stream(stream))
    _check("csa2_swa_merge", st)


def csa2_sparse_swa_decode_workspace_size(R, H, K):
    return int(lib().csa2_sparse_swa_decode_workspace_size(R, H, K))


def csa2_sparse_swa_decode(q_lat, codes, scales, idx, swa, swa_start, swa_len, softmax_scale, o, lse,
                           row_seq=None, workspace=None, stream=None):
    """Sparse attention over idx plus the window rows, one softmax: q_lat bf16 [R, H, 512];
    codes/scales [B, T, 256/32]; idx int32 [R, K]; swa bf16 [B, S, 512]; swa_start/swa_len int32 [R];
    o fp32 [R, H, 512]; lse fp32 [R, H]."""
    _need(q_lat, torch.bfloat16, "q_lat", 3)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _need(idx, torch.int32, "idx", 2)
    _need(swa, torch.bfloat16, "swa", 3)
    _need(swa_start, torch.int32, "swa_start", 1)
    _need(swa_len, torch.int32, "swa_len", 1)
    _need(o, torch.float32, "o", 3)
    _need(lse, torch.float32, "lse", 2)
    for t, nm in ((q_lat, "q_lat"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (swa, "swa"),
                  (swa_start, "swa_start"), (swa_len, "swa_len"), (o, "o"), (lse, "lse")):
        _dense(t, nm)
    R, H, C = q_lat.shape
    B, T, cb = codes.shape
    K = idx.shape[1]
    S = swa.shape[1]
    if C != 512 or cb != 256 or swa.shape != (B, S, 512) or o.shape != (R, H, 512) or lse.shape != (R, H):
        raise ValueError("sparse_swa_decode shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    need = csa2_sparse_swa_decode_workspace_size(R, H, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    st = lib().csa2_sparse_swa_decode(_p(q_lat), R, H, _p(codes), _p(scales), B, T, _p(row_seq), _p(idx), K,
                                      _p(swa), S, _p(swa_start), _p(swa_len), float(softmax_scale), _p(o), _p(lse),
                                      _p(workspace), workspace.numel(), _stream(stream))
    _check("csa2_sparse_swa_decode", st)


def csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K):
    return int(lib().csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K))


def _layers_shapes(q_lat, codes, scales, idx, layer_idx, swa, swa_start, swa_len, o, lse, row_seq):
    """Checks of the multi-layer attention arguments; returns L, R, H, B, T, K, S and the host layer_idx array."""
    _need(q_lat, torch.bfloat16, "q_lat", 4)
    _need(codes, torch.uint8, "codes", 3)
    _need(scales, torch.uint8, "scales", 3)
    _need(idx, torch.int32, "idx", 3)
    _need(swa, torch.bfloat16, "swa", 4)
    _need(swa_start, torch.int32, "swa_start", 2)
    _need(swa_len, torch.int32, "swa_len", 2)
    _need(o, torch.float32, "o", 4)
    _need(lse, torch.float32, "lse", 3)
    for t, nm in ((q_lat, "q_lat"), (codes, "codes"), (scales, "scales"), (idx, "idx"), (swa, "swa"),
                  (swa_start, "swa_start"), (swa_len, "swa_len"), (o, "o"), (lse, "lse")):
        _dense(t, nm)
    L, R, H, C = q_lat.shape
    B, T, cb = codes.shape
    n, Ri, K = idx.shape
    S = swa.shape[2]
    layer_idx = [int(v) for v in layer_idx]
    if (C != 512 or cb != 256 or Ri != R or len(layer_idx) != L or swa.shape != (L, B, S, 512)
            or swa_start.shape != (L, R) or swa_len.shape != (L, R) or o.shape != (L, R, H, 512)
            or lse.shape != (L, R, H)):
        raise ValueError("sparse_swa_decode_layers shapes")
    if any(v < 0 or v >= n for v in layer_idx):
        raise ValueError("layer_idx entries must select one of the idx slices")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    return L, R, H, B, T, K, S, (ctypes.c_int32 * L)(*layer_idx)


def csa2_sparse_swa_decode_layers(q_lat, codes, scales, idx, layer_idx, swa, swa_start, swa_len, softmax_scale, o,
                                  lse, row_seq=None, workspace=None, stream=None):
    """L layers of csa2_sparse_swa_decode in one launch: q_lat bf16 [L, R, H, 512]; idx int32 [n, R, K];
    layer_idx: L ints (host) selecting each layer's idx slice; swa bf16 [L, B, S, 512];
    swa_start/swa_len int32 [L, R]; o fp32 [L, R, H, 512]; lse fp32 [L, R, H]."""
    L, R, H, B, T, K, S, host_idx = _layers_shapes(q_lat, codes, scales, idx, layer_idx, swa, swa_start, swa_len, o,
                                                   lse, row_seq)
    need = csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_lat.device)
    st = lib().csa2_sparse_swa_decode_layers(L, _p(q_lat), R, H, _p(codes), _p(scales), B, T, _p(row_seq), _p(idx),
                                             ctypes.cast(host_idx, ctypes.c_void_p), K, _p(swa), S, _p(swa_start),
                                             _p(swa_len), float(softmax_scale), _p(o), _p(lse), _p(workspace),
                                             workspace.numel(), _stream(stream))
    _check("csa2_sparse_swa_decode_layers", st)


NOALLOC_SCRATCH_BYTES = 64 << 20


def csa2_sparse_swa_decode_layers_noalloc(q_lat, codes, scales, idx, layer_idx, swa, swa_start, swa_len,
                                          softmax_scale, o, lse, row_seq=None, stream=None):
    """csa2_sparse_swa_decode_layers with no workspace: the chunk partials go to the library's fixed
    64 MiB static device array (one per GPU, shared by every call on it).  Allocates no device memory."""
    L, R, H, B, T, K, S, host_idx = _layers_shapes(q_lat, codes, scales, idx, layer_idx, swa, swa_start, swa_len, o,
                                                   lse, row_seq)
    st = lib().csa2_sparse_swa_decode_layers_noalloc(L, _p(q_lat), R, H, _p(codes), _p(scales), B, T, _p(row_seq),
                                                     _p(idx), ctypes.cast(host_idx, ctypes.c_void_p), K, _p(swa), S,
                                                     _p(swa_start), _p(swa_len), float(softmax_scale), _p(o), _p(lse),
                                                     _stream(stream))
    _check("csa2_sparse_swa_decode_layers_noalloc", st)


def csa2_index_full_pool_workspace_size(R, T, k_pool):
    return int(lib().csa2_index_full_pool_workspace_size(R, T, k_pool))


def csa2_index_full_pool_batch_workspace_size(rows_per_batch, T, k_pool):
    """Workspace bytes for streaming batches of rows_per_batch rows (a larger workspace: fewer batches)."""
    return int(lib().csa2_index_full_pool_batch_workspace_size(rows_per_batch, T, k_pool))


def csa2_index_full_pool_streams(R, T):
    """True when csa2_index_full_pool selects during the scoring pass at R rows of T positions."""
    return bool(lib().csa2_index_full_pool_streams(R, T))


def csa2_index_full_pool(q_idx, k_idx, scores, k_pool, k_top, pool_idx, top_idx, pool_scores=None, row_seq=None,
                         row_limit=None, workspace=None, scan_events=None, stream=None):
    """Full-mode scores and the pool / Top-K selection in one call: q_idx uint8 [R, 64]; k_idx uint8 [B, T, 64];
    scores fp32 [R, T] (written) or None (not written: the selection needs no scores); pool_idx int32
    [R, k_pool]; top_idx int32 [R, k_top]; pool_scores fp32 [R, k_pool] or None.  scan_events: an optional (start, end) pair of already-created
    torch.cuda.Event objects, recorded by the library around the scoring kernel."""
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_idx, torch.uint8, "k_idx", 3)
    if scores is not None:
        _need(scores, torch.float32, "scores", 2)
        _dense(scores, "scores")
    _need(pool_idx, torch.int32, "pool_idx", 2)
    _need(top_idx, torch.int32, "top_idx", 2)
    for t, nm in ((q_idx, "q_idx"), (k_idx, "k_idx"), (pool_idx, "pool_idx"), (top_idx, "top_idx")):
        _dense(t, nm)
    R = q_idx.shape[0]
    B, T, d = k_idx.shape
    if q_idx.shape[1] != 64 or d != 64 or (scores is not None and scores.shape != (R, T)):
        raise ValueError("index_full_pool shapes")
    if pool_idx.shape != (R, k_pool) or top_idx.shape != (R, k_top):
        raise ValueError("pool_idx / top_idx shape")
    if pool_scores is not None:
        _need(pool_scores, torch.float32, "pool_scores", 2)
        _dense(pool_scores, "pool_scores")
        if pool_scores.shape != (R, k_pool):
            raise ValueError("pool_scores shape")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    if row_limit is not None:
        _need(row_limit, torch.int64, "row_limit", 1)
    need = csa2_index_full_pool_workspace_size(R, T, k_pool)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_idx.device)
    ev0 = ev1 = None
    if scan_events is not None:
        ev0, ev1 = (ctypes.c_void_p(int(e.cuda_event)) for e in scan_events)
        if not ev0.value or not ev1.value:
            raise ValueError("scan_events must be created (recorded once) before use")
    st = lib().csa2_index_full_pool(_p(q_idx), _p(k_idx), R, B, T, _p(row_seq), _p(row_limit), _p(scores), k_pool,
                                    k_top, _p(pool_idx), _p(pool_scores), _p(top_idx), _p(workspace),
                                    workspace.numel(), ev0, ev1, _stream(stream))
    _check("csa2_index_full_pool", st)


# ---------------------------------------------------------------------------
# paged global KV: pools of pages of `page` positions; block_table int32 [B, max_blocks]
# maps each sequence's logical block to its page (negative: unmapped)
# ---------------------------------------------------------------------------
def _table(block_table, page, T):
    _need(block_table, torch.int32, "block_table", 2)
    _dense(block_table, "block_table")
    return block_table.shape  # page size and capacity are checked by the library


def csa2_fp4_pack_rows(x, out_rows, codes, scales, stream=None):
    """x bf16 [n, C] (rows may be strided); out_rows int64 [n] (negative: skip); codes uint8 [N_rows, C/2] and
    scales uint8 [N_rows, C/16] (row-strided pools): row i of x is packed into row out_rows[i]."""
    _need(x, torch.bfloat16, "x", 2)
    _need(out_rows, torch.int64, "out_rows", 1)
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    n, C = x.shape
    if out_rows.shape != (n,) or codes.shape[1] != C // 2 or scales.shape[1] != C // 16:
        raise ValueError("pack_rows shapes")
    for t, nm in ((x, "x"), (codes, "codes"), (scales, "scales")):
        if t.stride(1) != 1:
            raise ValueError(f"{nm}: channels must be contiguous")
    _dense(out_rows, "out_rows")
    st = lib().csa2_fp4_pack_rows(_p(x), n, C, x.stride(0), _p(out_rows), _p(codes), codes.stride(0), _p(scales),
                                  scales.stride(0), _stream(stream))
    _check("csa2_fp4_pack_rows", st)


def csa2_index_full_paged(q_idx, k_pages, block_table, page, T, scores, row_seq=None, row_limit=None, stream=None):
    """csa2_index_full over paged keys: k_pages uint8 [n_pages * page, 64]; scores fp32 [R, T]."""
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_pages, torch.uint8, "k_pages", 2)
    _need(scores, torch.float32, "scores", 2)
    for t, nm in ((q_idx, "q_idx"), (k_pages, "k_pages"), (scores, "scores")):
        _dense(t, nm)
    B, max_blocks = _table(block_table, page, T)
    R = q_idx.shape[0]
    if q_idx.shape[1] != 64 or k_pages.shape[1] != 64 or scores.shape != (R, T):
        raise ValueError("index_full_paged shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    if row_limit is not None:
        _need(row_limit, torch.int64, "row_limit", 1)
    st = lib().csa2_index_full_paged(_p(q_idx), _p(k_pages), R, B, T, _p(row_seq), _p(row_limit), _p(block_table),
                                     max_blocks, page, _p(scores), _stream(stream))
    _check("csa2_index_full_paged", st)


def csa2_index_reindex_paged(q_idx, k_pages, block_table, page, T, pool, scores, row_seq=None, stream=None):
    """csa2_index_reindex over paged keys; pool int32 [R, P] of logical positions; scores fp32 [R, P]."""
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_pages, torch.uint8, "k_pages", 2)
    _need(pool, torch.int32, "pool", 2)
    _need(scores, torch.float32, "scores", 2)
    for t, nm in ((q_idx, "q_idx"), (k_pages, "k_pages"), (pool, "pool"), (scores, "scores")):
        _dense(t, nm)
    B, max_blocks = _table(block_table, page, T)
    R, P = pool.shape
    if scores.shape != (R, P) or q_idx.shape != (R, 64) or k_pages.shape[1] != 64:
        raise ValueError("reindex_paged shapes")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    st = lib().csa2_index_reindex_paged(_p(q_idx), _p(k_pages), R, B, T, _p(row_seq), _p(block_table), max_blocks,
                                        page, _p(pool), P, _p(scores), _stream(stream))
    _check("csa2_index_reindex_paged", st)


def csa2_index_full_pool_paged_workspace_size(R, T, k_pool):
    return int(lib().csa2_index_full_pool_paged_workspace_size(R, T, k_pool))


def csa2_index_full_pool_paged(q_idx, k_pages, block_table, page, T, scores, k_pool, k_top, pool_idx, top_idx,
                               pool_scores=None, row_seq=None, row_limit=None, workspace=None, stream=None):
    """csa2_index_full_pool over paged keys; scores fp32 [R, T] or None; outputs are logical positions."""
    _need(q_idx, torch.uint8, "q_idx", 2)
    _need(k_pages, torch.uint8, "k_pages", 2)
    if scores is not None:
        _need(scores, torch.float32, "scores", 2)
        _dense(scores, "scores")
    _need(pool_idx, torch.int32, "pool_idx", 2)
    _need(top_idx, torch.int32, "top_idx", 2)
    for t, nm in ((q_idx, "q_idx"), (k_pages, "k_pages"), (pool_idx, "pool_idx"), (top_idx, "top_idx")):
        _dense(t, nm)
    B, max_blocks = _table(block_table, page, T)
    R = q_idx.shape[0]
    if (q_idx.shape[1] != 64 or k_pages.shape[1] != 64 or (scores is not None and scores.shape != (R, T))
            or pool_idx.shape != (R, k_pool) or top_idx.shape != (R, k_top)):
        raise ValueError("index_full_pool_paged shapes")
    if pool_scores is not None:
        _need(pool_scores, torch.float32, "pool_scores", 2)
        _dense(pool_scores, "pool_scores")
        if pool_scores.shape != (R, k_pool):
            raise ValueError("pool_scores shape")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    if row_limit is not None:
        _need(row_limit, torch.int64, "row_limit", 1)
    if workspace is None:
        workspace = torch.empty(csa2_index_full_pool_paged_workspace_size(R, T, k_pool), dtype=torch.uint8,
                                device=q_idx.device)
    st = lib().csa2_index_full_pool_paged(_p(q_idx), _p(k_pages), R, B, T, _p(row_seq), _p(row_limit),
                                          _p(block_table), max_blocks, page, _p(scores), k_pool, k_top, _p(pool_idx),
                                          _p(pool_scores), _p(top_idx), _p(workspace), workspace.numel(),
                                          _stream(stream))
    _check("csa2_index_full_pool_paged", st)


def csa2_sparse_swa_decode_layers_paged(q_lat, code_pages, scale_pages, block_table, page, T, idx, layer_idx, swa,
                                        swa_start, swa_len, softmax_scale, o, lse, row_seq=None, workspace=None,
                                        stream=None):
    """csa2_sparse_swa_decode_layers over paged FP4 rows: code_pages uint8 [n_pages * page, 256], scale_pages
    uint8 [n_pages * page, 32]; idx holds logical positions."""
    _need(q_lat, torch.bfloat16, "q_lat", 4)
    _need(code_pages, torch.uint8, "code_pages", 2)
    _need(scale_pages, torch.uint8, "scale_pages", 2)
    _need(idx, torch.int32, "idx", 3)
    _need(swa, torch.bfloat16, "swa", 4)
    _need(swa_start, torch.int32, "swa_start", 2)
    _need(swa_len, torch.int32, "swa_len", 2)
    _need(o, torch.float32, "o", 4)
    _need(lse, torch.float32, "lse", 3)
    for t, nm in ((q_lat, "q_lat"), (code_pages, "code_pages"), (scale_pages, "scale_pages"), (idx, "idx"),
                  (swa, "swa"), (swa_start, "swa_start"), (swa_len, "swa_len"), (o, "o"), (lse, "lse")):
        _dense(t, nm)
    B, max_blocks = _table(block_table, page, T)
    L, R, H, C = q_lat.shape
    n, Ri, K = idx.shape
    S = swa.shape[2]
    layer_idx = [int(v) for v in layer_idx]
    if (C != 512 or code_pages.shape[1] != 256 or scale_pages.shape[1] != 32 or Ri != R or len(layer_idx) != L
            or swa.shape != (L, B, S, 512) or swa_start.shape != (L, R) or swa_len.shape != (L, R)
            or o.shape != (L, R, H, 512) or lse.shape != (L, R, H)):
        raise ValueError("sparse_swa_decode_layers_paged shapes")
    if any(v < 0 or v >= n for v in layer_idx):
        raise ValueError("layer_idx entries must select one of the idx slices")
    if row_seq is not None:
        _need(row_seq, torch.int32, "row_seq", 1)
    if workspace is None:
        workspace = torch.empty(csa2_sparse_swa_decode_layers_workspace_size(L, R, H, K), dtype=torch.uint8,
                                device=q_lat.device)
    host_idx = (ctypes.c_int32 * L)(*layer_idx)
    st = lib().csa2_sparse_swa_decode_layers_paged(L, _p(q_lat), R, H, _p(code_pages), _p(scale_pages), B, T,
                                                   _p(row_seq), _p(block_table), max_blocks, page, _p(idx),
                                                   ctypes.cast(host_idx, ctypes.c_void_p), K, _p(swa), S,
                                                   _p(swa_start), _p(swa_len), float(softmax_scale), _p(o), _p(lse),
                                                   _p(workspace), workspace.numel(), _stream(stream))
    _check("csa2_sparse_swa_decode_layers_paged", st)


def csa2_decode_append(new_latent, cache_rows, codes, scales, new_keys=None, k_idx=None, new_window=None, swa=None,
                       tok_pos=None, swa_start=None, swa_len=None, stream=None):
    """Decode-time append: new_latent bf16 [B, 512] packed into rows cache_rows (int64 [B]) of codes
    uint8 [N, 256] / scales uint8 [N, 32]; new_keys uint8 [B, 64] copied into those rows of k_idx uint8 [N, 64];
    new_window bf16 [L, B, 512] written into the mirrored window rings swa bf16 [L, B, S >= 256, 512] at
    position tok_pos (int64 [B]), with swa_start / swa_len int32 [L, B] updated."""
    _need(new_latent, torch.bfloat16, "new_latent", 2)
    _need(cache_rows, torch.int64, "cache_rows", 1)
    _need(codes, torch.uint8, "codes", 2)
    _need(scales, torch.uint8, "scales", 2)
    for t, nm in ((new_latent, "new_latent"), (cache_rows, "cache_rows"), (codes, "codes"), (scales, "scales")):
        _dense(t, nm)
    B = new_latent.shape[0]
    if new_latent.shape[1] != 512 or cache_rows.shape != (B,) or codes.shape[1] != 256 or scales.shape[1] != 32:
        raise ValueError("decode_append shapes")
    L, S = 0, 0
    if new_keys is not None:
        _need(new_keys, torch.uint8, "new_keys", 2)
        _need(k_idx, torch.uint8, "k_idx", 2)
        _dense(new_keys, "new_keys")
        _dense(k_idx, "k_idx")
        if new_keys.shape != (B, 64) or k_idx.shape[1] != 64:
            raise ValueError("key shapes")
    if new_window is not None:
        _need(new_window, torch.bfloat16, "new_window", 3)
        _need(swa, torch.bfloat16, "swa", 4)
        _need(tok_pos, torch.int64, "tok_pos", 1)
        _need(swa_start, torch.int32, "swa_start", 2)
        _need(swa_len, torch.int32, "swa_len", 2)
        for t, nm in ((new_window, "new_window"), (swa, "swa"), (tok_pos, "tok_pos"), (swa_start, "swa_start"),
                      (swa_len, "swa_len")):
            _dense(t, nm)
        L = new_window.shape[0]
        S = swa.shape[2]
        if (new_window.shape != (L, B, 512) or swa.shape != (L, B, S, 512) or tok_pos.shape != (B,)
                or swa_start.shape != (L, B) or swa_len.shape != (L, B)):
            raise ValueError("window shapes")
    st = lib().csa2_decode_append(B, L, _p(new_latent), _p(cache_rows), _p(codes), _p(scales), _p(new_keys),
                                  _p(k_idx), _p(new_window), _p(swa), S, _p(tok_pos), _p(swa_start), _p(swa_len),
                                  _stream(stream))
    _check("csa2_decode_append", st)


def csa2_absorb_q(q, w_uk, q_lat, stream=None):
    """Per-head queries into the latent space: q bf16 [R, H, 128], w_uk bf16 [H, 128, 512]
    -> q_lat bf16 [R, H, 512] (written)."""
    _need(q, torch.bfloat16, "q", 3)
    _need(w_uk, torch.bfloat16, "w_uk", 3)
    _need(q_lat, torch.bfloat16, "q_lat", 3)
    for t, nm in ((q, "q"), (w_uk, "w_uk"), (q_lat, "q_lat")):
        _dense(t, nm)
    R, H, D = q.shape
    if w_uk.shape != (H, D, 512) or q_lat.shape != (R, H, 512):
        raise ValueError("absorb shapes")
    _check("csa2_absorb_q", lib().csa2_absorb_q(_p(q), R, H, D, _p(w_uk), _p(q_lat), _stream(stream)))


def csa2_unabsorb_o(o_lat, w_uv, out, stream=None):
    """Latent attention outputs back to head space: o_lat fp32 [R, H, 512], w_uv bf16 [H, 128, 512]
    -> out fp32 [R, H, 128] (written)."""
    _need(o_lat, torch.float32, "o_lat", 3)
    _need(w_uv, torch.bfloat16, "w_uv", 3)
    _need(out, torch.float32, "out", 3)
    for t, nm in ((o_lat, "o_lat"), (w_uv, "w_uv"), (out, "out")):
        _dense(t, nm)
    R, H, C = o_lat.shape
    D = out.shape[2]
    if C != 512 or w_uv.shape != (H, D, 512) or out.shape[:2] != (R, H):
        raise ValueError("unabsorb shapes")
    _check("csa2_unabsorb_o", lib().csa2_unabsorb_o(_p(o_lat), R, H, D, _p(w_uv), _p(out), _stream(stream)))
