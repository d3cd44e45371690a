"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, its host-only functions agree bit-exactly with the oracle,
and invalid arguments are rejected before anything is launched (these calls
never reach the GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

c = pytest.importorskip("context_attention_varlen_amd")


def test_exports_match_header(root_dir):
    hdr = open(os.path.join(root_dir, "include", "cpattn.h")).read()
    declared = set(re.findall(r"\b(cpattn_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(c.EXPORTS)
    lib = ctypes.CDLL(c.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_device_info_rejects_bad_arguments():
    # argument checks come before any HIP call, so this runs without a GPU
    lib = c._lib
    out = ctypes.c_int32(0)
    assert lib.cpattn_device_info(0, None, ctypes.byref(out)) == c.ERR_INVALID_ARG
    assert lib.cpattn_device_info(0, ctypes.byref(out), None) == c.ERR_INVALID_ARG
    assert lib.cpattn_device_info(-1, ctypes.byref(out), ctypes.byref(out)) == c.ERR_INVALID_ARG


def test_fill_rejects_bad_arguments():
    # checked before any launch; count 0 enqueues nothing
    lib = c._lib
    assert lib.cpattn_fill_f32(None, 4, ctypes.c_float(0.0), None) == c.ERR_INVALID_ARG
    assert lib.cpattn_fill_f32(ctypes.c_void_p(16), -1, ctypes.c_float(0.0), None) == c.ERR_INVALID_ARG
    assert lib.cpattn_fill_f32(ctypes.c_void_p(20), 4, ctypes.c_float(0.0), None) == c.ERR_INVALID_ARG
    assert lib.cpattn_fill_f32(None, 0, ctypes.c_float(0.0), None) == c.OK


def test_version_and_status_strings():
    assert "gfx950" in c.cpattn_version()
    assert c.status_string(c.OK) == "ok"
    for s in (1, 2, 3, 4):
        assert c.status_string(s) != "ok"


@pytest.mark.parametrize("lens,cp", [([256], 4), ([64, 0, 192, 16], 4), ([40, 24, 8], 2), ([37, 5], 1),
                                     ([48, 16, 80, 8, 1024], 4), ([128, 64], 8)])
def test_partition_index_matches_oracle(lens, cp):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for r in range(cp):
        cu_l, l2g = c.cpattn_partition_index(cu, cp, r)
        cu_o, l2g_o, _, _ = oracle.local_rows(cu, cp, r)
        assert np.array_equal(cu_l, cu_o)
        assert np.array_equal(l2g, l2g_o)


def test_partition_index_full_configs():
    for name in ("long_video", "long_tail"):
        w = workloads.WORKLOADS[name]
        for r in (0, w.cp - 1):
            cu_l, l2g = c.cpattn_partition_index(w.cu_seqlens, w.cp, r)
            cu_o, l2g_o, _, _ = oracle.local_rows(w.cu_seqlens, w.cp, r)
            assert np.array_equal(cu_l, cu_o) and np.array_equal(l2g, l2g_o)


def test_partition_index_rejects_bad_input():
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index([0, 20], 4, 0)          # 20 % 8 != 0
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index([0, 16, 8], 2, 0)       # decreasing
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index([4, 16], 1, 0)          # cu[0] != 0
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index([0, 16], 2, 2)          # rank out of range


@pytest.mark.parametrize("lens,cp,mode,tf", [
    ([256], 4, 0, (0, 0)), ([64, 0, 192, 16], 4, 0, (0, 0)), ([40, 24, 8], 2, 1, (0, 0)),
    ([37, 5, 100], 1, 0, (0, 0)), ([96, 160], 2, 1, (0, 0)), ([2 * 3 * 37], 1, 2, (37, 3)),
    ([2 * 4 * 10, 2 * 4 * 10], 1, 2, (10, 4)), ([480, 32, 64], 8, 0, (0, 0))])
def test_count_pairs_matches_oracle_brute_force(lens, cp, mode, tf):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    for r in range(cp):
        for s in range(cp):
            n = c.cpattn_count_pairs(cu, mode, c.make_step(cp, r, s, *tf))
            assert n == oracle.count_pairs(cu, cp, r, s, mode, *tf)


def test_count_pairs_configs():
    W = workloads.WORKLOADS
    tot = lambda w, r: sum(c.cpattn_count_pairs(w.cu_seqlens, w.mask, c.make_step(w.cp, r, s, w.tf_chunk, w.tf_num))  # noqa
                           for s in range(w.cp))
    assert tot(W["tiny_fp32"], 0) == 8224
    assert tot(W["packed_varlen"], 0) == 22_395_656
    assert tot(W["long_video"], 0) == tot(W["long_video"], 7) == 4_294_983_680
    assert tot(W["tf_dit"], 0) == 1_518_566_400
    assert tot(W["long_tail"], 0) == tot(W["long_tail"], 3) == 304_747_728


class _FakeTensor:
    """Host-side stand-in with a data_ptr; the calls below fail validation
    before any device access."""
    is_cuda = True

    def __init__(self, shape, dtype, ptr=0x1000, strides=None):
        import torch
        self.shape = shape
        self.dtype = dtype
        self._ptr = ptr
        self._strides = strides or (shape[1] * shape[2], shape[2], 1)
        self.torch = torch

    def dim(self):
        return 3

    def stride(self, i):
        return self._strides[i]

    def data_ptr(self):
        return self._ptr

    def numel(self):
        return 1 << 20

    def element_size(self):
        return 1


def _fwd(q, k, v, out, step, mode=0, nseq=1, ws=None, cu=0x2000, lse=0x3000):
    import context_attention_varlen_amd as m
    ws = ws or _FakeTensor((1, 1, 1), None, ptr=0x4000)
    return m._lib.cpattn_fwd_step(ctypes.byref(m._tensor(q)), ctypes.byref(m._tensor(k)),
                                  ctypes.byref(m._tensor(v)), ctypes.c_void_p(cu), ctypes.c_void_p(cu), nseq,
                                  mode, ctypes.byref(step), 0.0, ctypes.byref(m._tensor(out)),
                                  ctypes.c_void_p(lse), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)


def test_fwd_step_rejects_bad_arguments():
    import torch
    bf = torch.bfloat16
    q = _FakeTensor((64, 4, 128), bf)
    kv = _FakeTensor((64, 2, 128), bf)
    st = c.make_step(1, 0, 0)
    assert _fwd(q, kv, kv, q, c.make_step(2, 2, 0)) == c.ERR_INVALID_ARG      # rank >= cp
    assert _fwd(q, kv, kv, q, c.make_step(2, 0, 2)) == c.ERR_INVALID_ARG      # step >= cp
    assert _fwd(q, _FakeTensor((64, 3, 128), bf), _FakeTensor((64, 3, 128), bf), q, st) == c.ERR_INVALID_ARG
    assert _fwd(_FakeTensor((64, 4, 96), bf), kv, kv, q, st) == c.ERR_UNSUPPORTED  # head_dim
    assert _fwd(q, _FakeTensor((64, 2, 128), torch.float32), kv, q, st) == c.ERR_INVALID_ARG  # mixed dtypes
    assert _fwd(_FakeTensor((64, 4, 128), bf, ptr=0x1008), kv, kv, q, st) == c.ERR_INVALID_ARG  # misaligned
    assert _fwd(q, kv, kv, q, st, cu=0) == c.ERR_INVALID_ARG                  # null cu_seqlens
    assert _fwd(q, kv, kv, q, st, mode=2) == c.ERR_INVALID_ARG                # TF without B, N
    assert _fwd(q, kv, kv, q, c.make_step(2, 0, 0, 8, 2), mode=2) == c.ERR_INVALID_ARG  # TF split, B < 32
    assert _fwd(q, kv, kv, q, c.make_step(4, 0, 0, 64, 6), mode=2) == c.ERR_INVALID_ARG  # TF split, N % cp
    assert _fwd(q, kv, kv, q, st, mode=7) == c.ERR_INVALID_ARG                # unknown mask
    small_ws = _FakeTensor((1, 1, 1), None, ptr=0x4000)
    small_ws.numel = lambda: 16
    assert _fwd(q, kv, kv, q, st, ws=small_ws) == c.ERR_WORKSPACE
    overlap = _FakeTensor((64, 4, 128), bf, strides=(128, 64, 1))
    assert _fwd(overlap, kv, kv, q, st) == c.ERR_INVALID_ARG                  # overlapping rows


def test_workspace_size_monotone():
    a = c.cpattn_workspace_size(1024, 1024, 4)
    b = c.cpattn_workspace_size(32768, 32768, 4)
    assert 0 < a < b and b % 256 == 0


@pytest.mark.parametrize("nseq,B,N,cp", [(1, 32, 4, 2), (3, 33, 6, 3), (2, 40, 12, 4), (1, 64, 12, 6), (2, 32, 8, 1)])
def test_partition_index_tf_matches_oracle(nseq, B, N, cp):
    """Balanced teacher-forcing split: host index plan bit-exact against the
    oracle's own split (cp = 1 is the identity)."""
    cu = np.arange(nseq + 1, dtype=np.int32) * (2 * B * N)
    for r in range(cp):
        cu_l, l2g = c.cpattn_partition_index_tf(cu, cp, r, B, N)
        cu_o, l2g_o, _, _ = oracle.tf_split.local_rows(cu, cp, r, B, N)
        assert np.array_equal(cu_l, cu_o)
        assert np.array_equal(l2g, l2g_o)


def test_count_pairs_tf_split_matches_oracle():
    B, N = 32, 12
    cu = np.array([0, 2 * B * N, 4 * B * N], np.int32)
    for cp in (2, 3, 4, 6):
        for r in range(cp):
            for s in range(cp):
                st = c.make_step(cp, r, s, B, N)
                assert c.cpattn_count_pairs(cu, oracle.TF_BLOCK, st) == oracle.tf_split.count_pairs(cu, cp, r, s, B, N)
    # every rank's total is N(N+1)B^2/cp per sequence when N is a multiple of 2*cp
    for cp in (2, 3, 6):
        for r in range(cp):
            tot = sum(c.cpattn_count_pairs(cu, oracle.TF_BLOCK, c.make_step(cp, r, s, B, N)) for s in range(cp))
            assert tot == 2 * N * (N + 1) * B * B // cp


def test_tf_split_rejects_bad_input():
    cu = np.array([0, 2 * 32 * 6], np.int32)
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index_tf(cu, 4, 0, 32, 6)          # 6 chunks over 4 ranks
    with pytest.raises(c.CpattnError):
        c.cpattn_partition_index_tf(cu, 2, 0, 32, 5)          # length is not 2*B*N
    with pytest.raises(c.CpattnError):
        c.cpattn_count_pairs(cu, oracle.TF_BLOCK, c.make_step(4, 0, 0, 32, 6))
    small = np.array([0, 2 * 16 * 4], np.int32)
    with pytest.raises(c.CpattnError):                        # chunk blocks below 32 rows at cp > 1
        c.cpattn_count_pairs(small, oracle.TF_BLOCK, c.make_step(2, 0, 0, 16, 4))


def _s2h(shards, group, dst):
    import context_attention_varlen_amd as m
    arr = (m.Tensor * len(shards))(*[m._tensor(t) for t in shards])
    return m._lib.cpattn_seq_to_head(arr, len(shards), group, ctypes.byref(m._tensor(dst)), None)


def test_ulysses_exchange_rejects_bad_input():
    import torch
    bf = torch.bfloat16
    sh = [_FakeTensor((64, 6, 128), bf, ptr=0x10000 + 0x100000 * i) for i in range(4)]
    dst = _FakeTensor((256, 2, 128), bf, ptr=0x900000)
    assert _s2h(sh, 0, dst) == c.ERR_INVALID_ARG                           # 6 heads, 4 groups
    assert _s2h(sh[:3], 3, dst) == c.ERR_INVALID_ARG                       # group out of range
    assert _s2h(sh[:3], 0, _FakeTensor((100, 2, 128), bf, ptr=0x900000)) == c.ERR_INVALID_ARG  # too few rows
    assert _s2h(sh[:3], 0, _FakeTensor((192, 2, 64), bf, ptr=0x900000)) == c.ERR_INVALID_ARG   # head_dim differs
    assert _s2h([], 0, dst) == c.ERR_INVALID_ARG                           # no shards


@pytest.mark.parametrize("H,W,cp", [(60, 104, 8), (64, 64, 8), (48, 48, 6), (12, 20, 4), (30, 32, 8), (7, 14, 2),
                                    (90, 160, 16), (5, 5, 1)])
def test_split_hw_matches_oracle(H, W, cp):
    assert c.cpattn_split_hw(H, W, cp) == oracle.hw_split.optimal_split(H, W, cp)


def test_split_hw_rejects_uneven():
    with pytest.raises(c.CpattnError):
        c.cpattn_split_hw(30, 30, 8)


@pytest.mark.parametrize("frames,H,W,cp,nseq", [(2, 4, 6, 4, 1), (3, 6, 4, 6, 2), (31, 30, 52, 8, 1), (1, 8, 8, 8, 2)])
def test_partition_index_hw_matches_oracle(frames, H, W, cp, nseq):
    split = c.cpattn_split_hw(H, W, cp)
    cu = np.arange(nseq + 1, dtype=np.int32) * (frames * H * W)
    for r in range(cp):
        cu_l, l2g = c.cpattn_partition_index_hw(cu, frames, H, W, split, r)
        cu_o, l2g_o, _, _ = oracle.hw_split.local_rows(cu, frames, H, W, split, r)
        assert np.array_equal(cu_l, cu_o)
        assert np.array_equal(l2g, l2g_o)


def test_count_pairs_bidir_any_split():
    """BIDIR at cp > 1 counts (L/cp)^2 per sequence and step for any split,
    also when L/cp is odd."""
    L = 31 * 30 * 52
    cu = np.array([0, L], np.int32)
    for s in range(8):
        assert c.cpattn_count_pairs(cu, oracle.BIDIR, c.make_step(8, 3, s)) == (L // 8) ** 2


def test_step_source_is_the_ring_rule():
    """(rank - step) mod cp for every rank and step; -1 for invalid steps."""
    for cp in (1, 2, 3, 4, 8):
        for r in range(cp):
            for s in range(cp):
                assert c.cpattn_step_source(c.make_step(cp, r, s)) == oracle.step_source(cp, r, s)
    for bad in (c.make_step(0, 0, 0), c.make_step(4, 4, 0), c.make_step(4, 0, 4), c.make_step(4, -1, 0)):
        with pytest.raises(c.CpattnError):
            c.cpattn_step_source(bad)


def test_binding_rejects_host_arrays_and_wrong_dtypes():
    """The binding checks what the raw-pointer arguments must be (device
    memory, int32 cu_seqlens of num_seqs + 1 entries, fp32 [H, T] LSE) before
    the C call; these raise without touching a GPU."""
    import torch
    with pytest.raises(ValueError):
        c._tensor(torch.zeros((4, 2, 64), dtype=torch.bfloat16))          # host memory
    cu64 = _FakeTensor((1, 1, 1), torch.int64)
    cu64.shape = (3,)
    with pytest.raises(ValueError):
        c._cu(cu64, "cu", 2)                                              # int64 cu_seqlens
    cu32 = _FakeTensor((1, 1, 1), torch.int32)
    cu32.shape = (4,)
    cu32.is_contiguous = lambda: True
    with pytest.raises(ValueError):
        c._cu(cu32, "cu", 2)                                              # num_seqs + 1 entries
    lse = _FakeTensor((1, 1, 1), torch.float32)
    lse.shape = (64, 4)
    lse.is_contiguous = lambda: True
    with pytest.raises(ValueError):
        c._f32(lse, "lse", (4, 64))                                       # [T, H] instead of [H, T]
    assert c._f32(lse, "lse", (64, 4)).value == lse.data_ptr()


def test_noalloc_forward_rejects_oversized_shapes():
    """The allocation-free forward refuses a shape whose schedule workspace
    exceeds the library's array before any HIP call (so this runs on CPU)."""
    import torch
    import context_attention_varlen_amd as m
    big = 4_000_000
    assert c.cpattn_workspace_size(big, big, 1) > (16 << 20)
    q = _FakeTensor((big, 1, 128), torch.bfloat16)
    st = c.make_step(1, 0, 0)
    rc = m._lib.cpattn_fwd_step_noalloc(ctypes.byref(m._tensor(q)), ctypes.byref(m._tensor(q)),
                                        ctypes.byref(m._tensor(q)), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x2000),
                                        1, 0, ctypes.byref(st), 0.0, ctypes.byref(m._tensor(q)),
                                        ctypes.c_void_p(0x3000), None)
    assert rc == c.ERR_WORKSPACE
