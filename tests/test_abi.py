"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import fp4_sparse_attention_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_header_functions_all_exported_and_bound():
    names = _header_functions()
    assert len(names) >= 12
    L = F.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(F.exported_symbols()) == names


def test_version_and_status_strings():
    assert F.csa2_abi_version() == 1
    L = F.lib()
    for s in range(7):
        assert L.csa2_status_str(s)
    assert b"unknown" in L.csa2_status_str(99)


NULL = None
DUMMY = ctypes.c_void_p(256)     # never dereferenced: every call below fails its host checks first


def test_pack_argument_errors():
    L = F.lib()
    assert L.csa2_fp4_pack(DUMMY, -1, 512, 512, DUMMY, 256, DUMMY, 32, NULL) == 1
    assert L.csa2_fp4_pack(DUMMY, 4, 500, 512, DUMMY, 256, DUMMY, 32, NULL) == 2
    assert L.csa2_fp4_pack(DUMMY, 4, 512, 100, DUMMY, 256, DUMMY, 32, NULL) == 1
    assert L.csa2_fp4_pack(DUMMY, 4, 512, 512, DUMMY, 100, DUMMY, 32, NULL) == 1
    assert L.csa2_fp4_pack(NULL, 4, 512, 512, DUMMY, 256, DUMMY, 32, NULL) == 1
    assert L.csa2_fp4_pack(ctypes.c_void_p(258), 4, 512, 512, DUMMY, 256, DUMMY, 32, NULL) == 3
    assert L.csa2_fp4_pack(DUMMY, 0, 512, 512, DUMMY, 256, DUMMY, 32, NULL) == 0      # empty: no-op
    assert L.csa2_fp4_unpack(DUMMY, DUMMY, 4, 48, DUMMY, NULL) == 2
    assert L.csa2_fp4_unpack(NULL, DUMMY, 4, 512, DUMMY, NULL) == 1


def test_index_argument_errors():
    L = F.lib()
    assert L.csa2_index_full(NULL, DUMMY, 1, 1, 64, NULL, NULL, DUMMY, NULL) == 1
    assert L.csa2_index_full(DUMMY, DUMMY, 2, 1, 64, NULL, NULL, DUMMY, NULL) == 1   # R != B, no row_seq
    assert L.csa2_index_full(DUMMY, DUMMY, 1, 1, 66, NULL, NULL, DUMMY, NULL) == 2   # T % 4
    assert L.csa2_index_full(DUMMY, DUMMY, 1, 1, 0, NULL, NULL, DUMMY, NULL) == 1
    assert L.csa2_index_reindex(DUMMY, DUMMY, 1, 1, 64, NULL, DUMMY, 6, DUMMY, NULL) == 2
    assert L.csa2_index_reindex(DUMMY, DUMMY, 1, 1, 64, NULL, NULL, 8, DUMMY, NULL) == 1


def test_topk_argument_errors_and_workspace():
    L = F.lib()
    ws = F.csa2_topk_workspace_size(8, 1 << 20, 2048)
    assert ws >= 8 * 2048 * 4
    assert F.csa2_topk_workspace_size(0, 10, 1) == 0
    assert L.csa2_topk(DUMMY, 1, 64, 64, 0, NULL, DUMMY, NULL, DUMMY, 1 << 20, NULL) == 1
    assert L.csa2_topk(DUMMY, 1, 62, 64, 8, NULL, DUMMY, NULL, DUMMY, 1 << 20, NULL) == 2
    assert L.csa2_topk(DUMMY, 1, 64, 60, 8, NULL, DUMMY, NULL, DUMMY, 1 << 20, NULL) == 1
    assert L.csa2_topk(DUMMY, 1, 64, 64, 8, NULL, DUMMY, NULL, DUMMY, 16, NULL) == 4
    assert L.csa2_topk(DUMMY, 1, 64, 64, 8, NULL, DUMMY, NULL, NULL, 1 << 20, NULL) == 4


def test_topk_pool_argument_errors():
    L = F.lib()
    ws = 1 << 20
    assert F.csa2_topk_pool_workspace_size(8, 1 << 20, 16384) == F.csa2_topk_workspace_size(8, 1 << 20, 16384)
    # k_top > k_pool, k_top <= 0, missing top_idx, small workspace
    assert L.csa2_topk_pool(DUMMY, 1, 64, 64, 8, 9, NULL, DUMMY, NULL, DUMMY, DUMMY, ws, NULL) == 1
    assert L.csa2_topk_pool(DUMMY, 1, 64, 64, 8, 0, NULL, DUMMY, NULL, DUMMY, DUMMY, ws, NULL) == 1
    assert L.csa2_topk_pool(DUMMY, 1, 64, 64, 8, 4, NULL, DUMMY, NULL, NULL, DUMMY, ws, NULL) == 1
    assert L.csa2_topk_pool(DUMMY, 1, 62, 64, 8, 4, NULL, DUMMY, NULL, DUMMY, DUMMY, ws, NULL) == 2
    assert L.csa2_topk_pool(DUMMY, 1, 64, 64, 8, 4, NULL, DUMMY, NULL, DUMMY, DUMMY, 16, NULL) == 4


def test_attention_argument_errors_and_workspace():
    L = F.lib()
    assert F.csa2_sparse_decode_workspace_size(64, 64, 2048) > 64 * 64 * 512 * 4
    assert F.csa2_swa_merge_workspace_size(8, 64) >= 8 * 64 * 512 * 4
    assert F.csa2_sparse_swa_decode_workspace_size(8, 64, 2048) >= F.csa2_sparse_decode_workspace_size(8, 64, 2048)
    assert F.csa2_sparse_swa_decode_layers_workspace_size(4, 8, 64, 2048) >= \
        4 * F.csa2_sparse_swa_decode_workspace_size(8, 64, 2048) // 2
    assert F.csa2_sparse_swa_decode_layers_workspace_size(9, 8, 64, 2048) == 0
    args = [DUMMY, 1, 64, DUMMY, DUMMY, 1, 4096, NULL, DUMMY, 256, 0.1, DUMMY, DUMMY, DUMMY, 1 << 30, NULL]
    bad_h = list(args); bad_h[2] = 20
    assert L.csa2_sparse_decode(*bad_h) == 2
    bad_k = list(args); bad_k[9] = 0
    assert L.csa2_sparse_decode(*bad_k) == 1
    small_ws = list(args); small_ws[14] = 100
    assert L.csa2_sparse_decode(*small_ws) == 4
    no_seq = list(args); no_seq[1] = 2
    assert L.csa2_sparse_decode(*no_seq) == 1
    sargs = [DUMMY, 1, 64, DUMMY, 1, 128, NULL, DUMMY, DUMMY, 0.1, DUMMY, NULL, DUMMY, NULL, DUMMY, 1 << 30, NULL]
    assert L.csa2_swa_merge(*sargs) == 1          # o_sparse without lse_sparse
    sargs[10] = NULL
    sargs[1] = 1
    sargs[2] = 8
    assert L.csa2_swa_merge(*sargs) == 2          # H = 8


def test_no_cpu_fallback_in_binding():
    # the binding refuses CPU tensors instead of computing anything itself
    import torch
    x = torch.zeros((4, 512), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        F.csa2_fp4_pack(x, torch.zeros((4, 256), dtype=torch.uint8), torch.zeros((4, 32), dtype=torch.uint8))


def test_layers_call_argument_errors():
    L = F.lib()
    good = (ctypes.c_int32 * 4)(0, 1, 1, 1)
    bad = (ctypes.c_int32 * 4)(0, -1, 1, 1)
    args = [4, DUMMY, 8, 64, DUMMY, DUMMY, 8, 1 << 20, NULL, DUMMY, ctypes.cast(good, ctypes.c_void_p), 2048, DUMMY, 128,
            DUMMY, DUMMY, 0.1, DUMMY, DUMMY, DUMMY, 1 << 30, NULL]
    a = list(args); a[10] = ctypes.cast(bad, ctypes.c_void_p)
    assert L.csa2_sparse_swa_decode_layers(*a) == 1          # negative layer_idx entry
    a = list(args); a[10] = NULL
    assert L.csa2_sparse_swa_decode_layers(*a) == 1          # no layer_idx
    a = list(args); a[0] = 9
    assert L.csa2_sparse_swa_decode_layers(*a) == 2          # more than 8 layers
    a = list(args); a[3] = 20
    assert L.csa2_sparse_swa_decode_layers(*a) == 2          # H = 20
    a = list(args); a[20] = 100
    assert L.csa2_sparse_swa_decode_layers(*a) == 4          # workspace too small


def test_noalloc_call_argument_errors():
    # the allocation-free layers call refuses a shape whose partials exceed its static array before
    # touching the GPU, and checks its other arguments like the workspace call
    L = F.lib()
    one = (ctypes.c_int32 * 1)(0)
    args = [1, DUMMY, 128, 64, DUMMY, DUMMY, 1, 8192, DUMMY, DUMMY, ctypes.cast(one, ctypes.c_void_p), 8192, DUMMY,
            128, DUMMY, DUMMY, 0.1, DUMMY, DUMMY, NULL]
    assert F.csa2_sparse_swa_decode_layers_workspace_size(1, 128, 64, 8192) > F.NOALLOC_SCRATCH_BYTES
    assert L.csa2_sparse_swa_decode_layers_noalloc(*args) == 6
    a = list(args); a[10] = NULL
    assert L.csa2_sparse_swa_decode_layers_noalloc(*a) == 1
    a = list(args); a[3] = 20
    assert L.csa2_sparse_swa_decode_layers_noalloc(*a) == 2
    a = list(args); a[1] = NULL
    assert L.csa2_sparse_swa_decode_layers_noalloc(*a) == 1
    assert F.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_index_full_pool_argument_errors():
    L = F.lib()
    ws = 1 << 20
    base = [DUMMY, DUMMY, 1, 1, 4096, NULL, NULL, DUMMY, 16, 4, DUMMY, NULL, DUMMY, DUMMY, ws, NULL, NULL, NULL]
    a = list(base); a[9] = 17
    assert L.csa2_index_full_pool(*a) == 1        # k_top > k_pool
    a = list(base); a[12] = NULL
    assert L.csa2_index_full_pool(*a) == 1        # no top_idx
    a = list(base); a[4] = 4098
    assert L.csa2_index_full_pool(*a) == 2        # T % 4
    a = list(base); a[2] = 2
    assert L.csa2_index_full_pool(*a) == 1        # R != B without row_seq
    a = list(base); a[14] = 16
    assert L.csa2_index_full_pool(*a) == 4        # workspace
    # streaming shapes (rows longer than 32,768): room for the candidate blocks of one batch of rows; the
    # size query keeps every shape below 1 GB (row batches), a single batch takes R x T x 8 bytes and more
    assert F.csa2_index_full_pool_workspace_size(8, 1 << 20, 16384) >= 8 * (1 << 20) * 8
    for R, T in ((4096, 1 << 18), (4096, 1 << 20), (5000, 1 << 18), (65536, 1 << 21)):
        assert F.csa2_index_full_pool_streams(R, T)
        assert F.csa2_index_full_pool_workspace_size(R, T, 2048) < 10 ** 9
        assert F.csa2_index_full_pool_batch_workspace_size(R, T, 2048) >= R * T * 8
    assert not F.csa2_index_full_pool_streams(64, 1 << 15)
    # shapes that select from scores get room for the scores the caller may not take
    assert (F.csa2_index_full_pool_workspace_size(64, 1 << 15, 2048)
            >= F.csa2_topk_workspace_size(64, 1 << 15, 2048) + 64 * (1 << 15) * 4)
    # scores may be null: the argument checks still run (and fail here on the workspace, before any launch)
    a = list(base); a[7] = NULL; a[14] = 16
    assert L.csa2_index_full_pool(*a) == 4


def test_paged_argument_errors():
    L = F.lib()
    # page map: null table / max_blocks <= 0 / page <= 0 -> EINVAL; page % 128, T > capacity -> ESHAPE
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 1, 1, 256, NULL, NULL, NULL, 2, 128, DUMMY, NULL) == 1
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 1, 1, 256, NULL, NULL, DUMMY, 0, 128, DUMMY, NULL) == 1
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 1, 1, 256, NULL, NULL, DUMMY, 2, 0, DUMMY, NULL) == 1
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 1, 1, 256, NULL, NULL, DUMMY, 2, 192, DUMMY, NULL) == 2
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 1, 1, 384, NULL, NULL, DUMMY, 2, 128, DUMMY, NULL) == 2
    assert L.csa2_index_full_paged(DUMMY, DUMMY, 2, 1, 256, NULL, NULL, DUMMY, 2, 128, DUMMY, NULL) == 1
    assert L.csa2_index_reindex_paged(DUMMY, DUMMY, 1, 1, 256, NULL, DUMMY, 1, 128, DUMMY, 8, DUMMY, NULL) == 2
    assert L.csa2_index_reindex_paged(DUMMY, DUMMY, 1, 1, 256, NULL, NULL, 2, 128, DUMMY, 8, DUMMY, NULL) == 1
    ws = F.csa2_index_full_pool_paged_workspace_size(1, 4096, 512)
    assert ws == F.csa2_index_full_pool_workspace_size(1, 4096, 512)
    assert L.csa2_index_full_pool_paged(DUMMY, DUMMY, 1, 1, 4096, NULL, NULL, DUMMY, 8, 256, DUMMY, 512, 64,
                                        DUMMY, NULL, DUMMY, DUMMY, ws, NULL) == 2        # 8 x 256 < 4096
    assert L.csa2_index_full_pool_paged(DUMMY, DUMMY, 1, 1, 4096, NULL, NULL, NULL, 16, 256, DUMMY, 512, 64,
                                        DUMMY, NULL, DUMMY, DUMMY, ws, NULL) == 1
    assert L.csa2_index_full_pool_paged(DUMMY, DUMMY, 1, 1, 4096, NULL, NULL, DUMMY, 16, 256, DUMMY, 512, 64,
                                        DUMMY, NULL, DUMMY, DUMMY, 16, NULL) == 4        # workspace too small
    # scattered pack: output-row list must be given (and 8-byte aligned)
    assert L.csa2_fp4_pack_rows(DUMMY, 2, 512, 512, NULL, DUMMY, 256, DUMMY, 32, NULL) == 1
    assert L.csa2_fp4_pack_rows(DUMMY, 2, 512, 512, ctypes.c_void_p(260), DUMMY, 256, DUMMY, 32, NULL) == 3
    assert L.csa2_fp4_pack_rows(DUMMY, 2, 500, 512, DUMMY, DUMMY, 256, DUMMY, 32, NULL) == 2
    assert L.csa2_fp4_pack_rows(DUMMY, 0, 512, 512, NULL, NULL, 256, NULL, 32, NULL) == 0
    # attention over pages: null table, then a page size off the quantum
    host_idx = (ctypes.c_int32 * 1)(0)
    args = lambda table, page: (1, DUMMY, 1, 64, DUMMY, DUMMY, 1, 256, NULL, table, 2, page, DUMMY,
                                ctypes.cast(host_idx, ctypes.c_void_p), 64, DUMMY, 128, DUMMY, DUMMY,
                                ctypes.c_float(0.05), DUMMY, DUMMY, DUMMY, 1 << 30, NULL)
    assert L.csa2_sparse_swa_decode_layers_paged(*args(NULL, 128)) == 1
    assert L.csa2_sparse_swa_decode_layers_paged(*args(DUMMY, 100)) == 2


def test_decode_append_argument_errors():
    L = F.lib()
    assert L.csa2_decode_append(-1, 0, DUMMY, DUMMY, DUMMY, DUMMY, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) == 1
    assert L.csa2_decode_append(0, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) == 0
    assert L.csa2_decode_append(2, 0, NULL, DUMMY, DUMMY, DUMMY, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) == 1
    assert L.csa2_decode_append(2, 0, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) == 1
    # a window row without layers, then a ring shorter than two windows
    assert L.csa2_decode_append(2, 0, DUMMY, DUMMY, DUMMY, DUMMY, NULL, NULL, DUMMY, DUMMY, 256, DUMMY, DUMMY, DUMMY,
                                NULL) == 1
    assert L.csa2_decode_append(2, 3, DUMMY, DUMMY, DUMMY, DUMMY, NULL, NULL, DUMMY, DUMMY, 128, DUMMY, DUMMY, DUMMY,
                                NULL) == 2
    assert L.csa2_decode_append(2, 0, ctypes.c_void_p(264), DUMMY, DUMMY, DUMMY, NULL, NULL, NULL, NULL, 0, NULL, NULL,
                                NULL, NULL) == 3


def test_absorb_argument_errors():
    L = F.lib()
    assert L.csa2_absorb_q(NULL, 1, 4, 128, NULL, NULL, NULL) == 1                 # null pointers
    assert L.csa2_absorb_q(DUMMY, -1, 4, 128, DUMMY, DUMMY, NULL) == 1             # R < 0
    assert L.csa2_absorb_q(DUMMY, 1, 0, 128, DUMMY, DUMMY, NULL) == 1              # H <= 0
    assert L.csa2_absorb_q(DUMMY, 1, 4, 64, DUMMY, DUMMY, NULL) == 2               # D != 128
    assert L.csa2_absorb_q(ctypes.c_void_p(264), 1, 4, 128, DUMMY, DUMMY, NULL) == 3
    assert L.csa2_absorb_q(DUMMY, 0, 4, 128, DUMMY, DUMMY, NULL) == 0              # empty: no-op
    assert L.csa2_unabsorb_o(NULL, 1, 4, 128, DUMMY, DUMMY, NULL) == 1
    assert L.csa2_unabsorb_o(DUMMY, 1, 4, 96, DUMMY, DUMMY, NULL) == 2
    assert L.csa2_unabsorb_o(DUMMY, 1, 4, 128, DUMMY, ctypes.c_void_p(260), NULL) == 3
    assert L.csa2_unabsorb_o(DUMMY, 0, 4, 128, DUMMY, DUMMY, NULL) == 0
