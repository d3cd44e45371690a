"""Python binding of libcpattn (blockwise zigzag-ring varlen attention on
MI355X).  Argument marshalling only: every step of the path runs in the HIP
kernels of libcpattn.so; torch supplies device memory and the stream.

The functions carry the names of the C entry points in include/cpattn.h.
Tensors are THD torch tensors ([tokens, heads, head_dim], head_dim
contiguous); LSE / delta arrays are fp32 [heads, tokens]; fp32 accumulators
are dense [tokens, heads, head_dim].  A non-zero status raises CpattnError.

There is no fallback: if libcpattn.so is missing or fails to load, importing
this package raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

CAUSAL, BIDIR, TF_BLOCK = 0, 1, 2
F32, BF16 = 0, 1
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_INFEASIBLE, ERR_NOMEM = 0, 1, 2, 3, 4, 5, 6

EXPORTS = (
    "cpattn_version", "cpattn_status_string", "cpattn_last_hip_error", "cpattn_device_info", "cpattn_partition_index", "cpattn_partition",
    "cpattn_unpartition", "cpattn_partition_index_tf", "cpattn_partition_tf", "cpattn_unpartition_tf",
    "cpattn_seq_to_head", "cpattn_head_to_seq", "cpattn_split_hw", "cpattn_partition_index_hw",
    "cpattn_partition_hw", "cpattn_unpartition_hw",
    "cpattn_count_pairs", "cpattn_step_source", "cpattn_workspace_size", "cpattn_workspace_status",
    "cpattn_fwd_step", "cpattn_fwd_step_noalloc", "cpattn_merge", "cpattn_fill_f32", "cpattn_bwd_preprocess", "cpattn_bwd_step",
    "cpattn_dcp_plan_batch", "cpattn_dcp_quotas",
)


class CpattnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {status_string(status)} (status {status})"
        if status == ERR_HIP:
            msg += f": {_lib.cpattn_last_hip_error().decode()}"
        super().__init__(msg)


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("tokens", ctypes.c_int64),
                ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("stride_token", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class DcpConfig(ctypes.Structure):
    _fields_ = [("gpus", ctypes.c_int32), ("max_cp", ctypes.c_int32), ("pp", ctypes.c_int32),
                ("vpp", ctypes.c_int32), ("mem_tokens", ctypes.c_int64), ("work_quad", ctypes.c_int64),
                ("work_lin", ctypes.c_int64), ("m_min", ctypes.c_int32), ("m_max", ctypes.c_int32),
                ("knee_radius", ctypes.c_int32)]


class DcpPlan(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("knee", ctypes.c_int32), ("num_buckets", ctypes.c_int32),
                ("step_time", ctypes.c_double), ("sample_bucket", ctypes.c_void_p),
                ("bucket_cp", ctypes.c_void_p), ("bucket_slot", ctypes.c_void_p),
                ("bucket_rank", ctypes.c_void_p), ("bucket_tokens", ctypes.c_void_p),
                ("bucket_load", ctypes.c_void_p), ("times", ctypes.c_void_p), ("budget", ctypes.c_void_p),
                ("bucket_capacity", ctypes.c_int32)]


class Step(ctypes.Structure):
    _fields_ = [("cp", ctypes.c_int32), ("rank", ctypes.c_int32), ("step", ctypes.c_int32),
                ("tf_chunk_tokens", ctypes.c_int32), ("tf_num_chunks", ctypes.c_int32)]


def _load():
    # torch ships its own HIP runtime (libamdhip64).  Load it first so that
    # libcpattn binds to the same runtime instance: the stream handles and
    # device pointers torch hands over are only meaningful there, and two
    # runtimes in one process do not share the device.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libcpattn.so not built at {LIB_PATH}; run python context_attention_varlen_amd/build.py "
                          "(by path: importing the package needs the library)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    TP = ctypes.POINTER(Tensor)
    SP = ctypes.POINTER(Step)
    sig = {
        "cpattn_version": (ctypes.c_char_p, []),
        "cpattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "cpattn_last_hip_error": (ctypes.c_char_p, []),
        "cpattn_device_info": (ctypes.c_int, [I32, P, P]),
        "cpattn_partition_index": (ctypes.c_int, [P, I32, I32, I32, P, P]),
        "cpattn_partition": (ctypes.c_int, [TP, TP, P, I32, I32, I32, P]),
        "cpattn_unpartition": (ctypes.c_int, [TP, TP, P, I32, I32, I32, P]),
        "cpattn_partition_index_tf": (ctypes.c_int, [P, I32, I32, I32, I32, I32, P, P]),
        "cpattn_partition_tf": (ctypes.c_int, [TP, TP, P, I32, I32, I32, I32, I32, P]),
        "cpattn_unpartition_tf": (ctypes.c_int, [TP, TP, P, I32, I32, I32, I32, I32, P]),
        "cpattn_seq_to_head": (ctypes.c_int, [TP, I32, I32, TP, P]),
        "cpattn_split_hw": (ctypes.c_int, [I32, I32, I32, P, P]),
        "cpattn_partition_index_hw": (ctypes.c_int, [P, I32, I32, I32, I32, I32, I32, I32, P, P]),
        "cpattn_partition_hw": (ctypes.c_int, [TP, TP, P, I32, I32, I32, I32, I32, I32, I32, P]),
        "cpattn_unpartition_hw": (ctypes.c_int, [TP, TP, P, I32, I32, I32, I32, I32, I32, I32, P]),
        "cpattn_head_to_seq": (ctypes.c_int, [TP, I32, I32, TP, P]),
        "cpattn_count_pairs": (I64, [P, I32, ctypes.c_int, SP]),
        "cpattn_step_source": (I32, [SP]),
        "cpattn_workspace_size": (S, [I64, I64, I32]),
        "cpattn_workspace_status": (ctypes.c_int, [P, P, ctypes.POINTER(ctypes.c_int)]),
        "cpattn_fwd_step": (ctypes.c_int, [TP, TP, TP, P, P, I32, ctypes.c_int, SP, F, TP, P, P, S, P]),
        "cpattn_fwd_step_noalloc": (ctypes.c_int, [TP, TP, TP, P, P, I32, ctypes.c_int, SP, F, TP, P, P]),
        "cpattn_merge": (ctypes.c_int, [P, P, TP, P, P]),
        "cpattn_fill_f32": (ctypes.c_int, [P, I64, F, P]),
        "cpattn_bwd_preprocess": (ctypes.c_int, [P, TP, P, P]),
        "cpattn_bwd_step": (ctypes.c_int, [TP, TP, TP, TP, P, P, P, P, I32, ctypes.c_int, SP, F,
                                           P, P, P, P, S, P]),
        "cpattn_dcp_plan_batch": (ctypes.c_int, [P, I32, ctypes.POINTER(DcpConfig), ctypes.POINTER(DcpPlan)]),
        "cpattn_dcp_quotas": (ctypes.c_int, [P, I32, I32, I32, ctypes.c_double, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def status_string(status: int) -> str:
    return _lib.cpattn_status_string(int(status)).decode()


def _check(status, where):
    if status != OK:
        raise CpattnError(status, where)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensor(t) -> Tensor:
    if t.dim() != 3:
        raise ValueError("THD tensors are [tokens, heads, head_dim]")
    if t.stride(2) != 1:
        raise ValueError("head_dim must be contiguous")
    if not t.is_cuda:
        raise ValueError("THD tensors must be in device memory")
    return Tensor(t.data_ptr(), _dtype_code(t), t.shape[0], t.shape[1], t.shape[2], t.stride(0), t.stride(1))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# The C ABI takes raw pointers for these arrays; what their declarations in
# cpattn.h require is checked here so that a wrong torch dtype, device, shape
# or layout raises instead of reaching the device.
def _dev_array(t, name, dtype, shape):
    import torch
    if t is None:
        raise ValueError(f"{name}: missing")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be in device memory")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    del torch


def _cu(t, name, num_seqs):
    import torch
    _dev_array(t, name, torch.int32, (num_seqs + 1,))
    return _ptr(t)


def _f32(t, name, shape):
    import torch
    _dev_array(t, name, torch.float32, shape)
    return _ptr(t)


def _workspace(t):
    if t is None or not t.is_cuda or not t.is_contiguous():
        raise ValueError("workspace: a contiguous device tensor")
    return _ptr(t), t.numel() * t.element_size()


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_step(cp, rank, step, tf_chunk_tokens=0, tf_num_chunks=0) -> Step:
    return Step(cp, rank, step, tf_chunk_tokens, tf_num_chunks)


# ---------------------------------------------------------------------------
# entry points (names as in include/cpattn.h)
# ---------------------------------------------------------------------------
def cpattn_version() -> str:
    return _lib.cpattn_version().decode()


def cpattn_device_info(device: int = 0):
    """(compute units, peak shader clock in kHz) of a HIP device."""
    cus, khz = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.cpattn_device_info(int(device), ctypes.byref(cus), ctypes.byref(khz)), "cpattn_device_info")
    return cus.value, khz.value


def cpattn_partition_index(cu_seqlens_global, cp: int, rank: int, with_map: bool = True):
    """Host index plan: (cu_seqlens_local int32, local_to_global int64 or None)."""
    cu = np.ascontiguousarray(cu_seqlens_global, dtype=np.int32)
    nseq = len(cu) - 1
    cu_l = np.zeros(nseq + 1, np.int32)
    l2g = np.zeros(int(cu[-1]) // cp if nseq >= 0 else 0, np.int64) if with_map else None
    st = _lib.cpattn_partition_index(cu.ctypes.data, nseq, cp, rank, cu_l.ctypes.data,
                                     l2g.ctypes.data if l2g is not None else None)
    _check(st, "cpattn_partition_index")
    return cu_l, l2g


def cpattn_partition(src_global, dst_local, cu_seqlens_global_dev, num_seqs, cp, rank, stream=None):
    st = _lib.cpattn_partition(ctypes.byref(_tensor(src_global)), ctypes.byref(_tensor(dst_local)),
                               _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, cp, rank, _stream(stream))
    _check(st, "cpattn_partition")


def cpattn_unpartition(src_local, dst_global, cu_seqlens_global_dev, num_seqs, cp, rank, stream=None):
    st = _lib.cpattn_unpartition(ctypes.byref(_tensor(src_local)), ctypes.byref(_tensor(dst_global)),
                                 _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, cp, rank, _stream(stream))
    _check(st, "cpattn_unpartition")


def cpattn_partition_index_tf(cu_seqlens_global, cp: int, rank: int, tf_chunk_tokens: int, tf_num_chunks: int,
                              with_map: bool = True):
    """Host index plan of the balanced teacher-forcing split: (cu_seqlens_local
    int32, local_to_global int64 or None)."""
    cu = np.ascontiguousarray(cu_seqlens_global, dtype=np.int32)
    nseq = len(cu) - 1
    cu_l = np.zeros(nseq + 1, np.int32)
    l2g = np.zeros(int(cu[-1]) // cp if nseq >= 0 else 0, np.int64) if with_map else None
    st = _lib.cpattn_partition_index_tf(cu.ctypes.data, nseq, cp, rank, tf_chunk_tokens, tf_num_chunks,
                                        cu_l.ctypes.data, l2g.ctypes.data if l2g is not None else None)
    _check(st, "cpattn_partition_index_tf")
    return cu_l, l2g


def cpattn_partition_tf(src_global, dst_local, cu_seqlens_global_dev, num_seqs, cp, rank, tf_chunk_tokens,
                        tf_num_chunks, stream=None):
    st = _lib.cpattn_partition_tf(ctypes.byref(_tensor(src_global)), ctypes.byref(_tensor(dst_local)),
                                  _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, cp, rank, tf_chunk_tokens, tf_num_chunks,
                                  _stream(stream))
    _check(st, "cpattn_partition_tf")


def cpattn_unpartition_tf(src_local, dst_global, cu_seqlens_global_dev, num_seqs, cp, rank, tf_chunk_tokens,
                          tf_num_chunks, stream=None):
    st = _lib.cpattn_unpartition_tf(ctypes.byref(_tensor(src_local)), ctypes.byref(_tensor(dst_global)),
                                    _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, cp, rank, tf_chunk_tokens, tf_num_chunks,
                                    _stream(stream))
    _check(st, "cpattn_unpartition_tf")


def cpattn_split_hw(H, W, cp):
    """(split_h, split_w): the even height/width split of cp closest to square tiles."""
    sh, sw = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(_lib.cpattn_split_hw(H, W, cp, ctypes.byref(sh), ctypes.byref(sw)), "cpattn_split_hw")
    return sh.value, sw.value


def cpattn_partition_index_hw(cu_seqlens_global, frames, H, W, split, rank, with_map: bool = True):
    """Host index plan of the height/width split: (cu_seqlens_local, local_to_global or None)."""
    cu = np.ascontiguousarray(cu_seqlens_global, dtype=np.int32)
    nseq = len(cu) - 1
    cp = split[0] * split[1]
    cu_l = np.zeros(nseq + 1, np.int32)
    l2g = np.zeros(int(cu[-1]) // cp if nseq >= 0 else 0, np.int64) if with_map else None
    st = _lib.cpattn_partition_index_hw(cu.ctypes.data, nseq, frames, H, W, split[0], split[1], rank,
                                        cu_l.ctypes.data, l2g.ctypes.data if l2g is not None else None)
    _check(st, "cpattn_partition_index_hw")
    return cu_l, l2g


def cpattn_partition_hw(src_global, dst_local, cu_seqlens_global_dev, num_seqs, frames, H, W, split, rank,
                        stream=None):
    st = _lib.cpattn_partition_hw(ctypes.byref(_tensor(src_global)), ctypes.byref(_tensor(dst_local)),
                                  _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, frames, H, W, split[0], split[1], rank,
                                  _stream(stream))
    _check(st, "cpattn_partition_hw")


def cpattn_unpartition_hw(src_local, dst_global, cu_seqlens_global_dev, num_seqs, frames, H, W, split, rank,
                          stream=None):
    st = _lib.cpattn_unpartition_hw(ctypes.byref(_tensor(src_local)), ctypes.byref(_tensor(dst_global)),
                                    _cu(cu_seqlens_global_dev, "cu_seqlens_global", num_seqs), num_seqs, frames, H, W, split[0], split[1], rank,
                                    _stream(stream))
    _check(st, "cpattn_unpartition_hw")


def cpattn_seq_to_head(shards, group, gathered, stream=None):
    """Head group `group` of every shard (list of [T_s, H, d] tensors, rank
    order) into gathered [sum T_s, H/len(shards), d]."""
    arr = (Tensor * len(shards))(*[_tensor(t) for t in shards])
    st = _lib.cpattn_seq_to_head(arr, len(shards), group, ctypes.byref(_tensor(gathered)), _stream(stream))
    _check(st, "cpattn_seq_to_head")


def cpattn_head_to_seq(gathered, group, shards, stream=None):
    """Inverse of cpattn_seq_to_head: writes head group `group` back into the shards."""
    arr = (Tensor * len(shards))(*[_tensor(t) for t in shards])
    st = _lib.cpattn_head_to_seq(ctypes.byref(_tensor(gathered)), len(shards), group, arr, _stream(stream))
    _check(st, "cpattn_head_to_seq")


def cpattn_count_pairs(cu_seqlens_global, mask_mode, step: Step) -> int:
    cu = np.ascontiguousarray(cu_seqlens_global, dtype=np.int32)
    n = _lib.cpattn_count_pairs(cu.ctypes.data, len(cu) - 1, mask_mode, ctypes.byref(step))
    if n < 0:
        raise CpattnError(ERR_INVALID_ARG, "cpattn_count_pairs")
    return int(n)


def cpattn_step_source(step: Step) -> int:
    """Rank whose K/V share the step uses: (rank - step) mod cp."""
    j = _lib.cpattn_step_source(ctypes.byref(step))
    if j < 0:
        raise CpattnError(ERR_INVALID_ARG, "cpattn_step_source")
    return int(j)


def cpattn_workspace_size(tokens_q, tokens_k, num_seqs) -> int:
    return int(_lib.cpattn_workspace_size(tokens_q, tokens_k, num_seqs))


def cpattn_workspace_status(workspace, stream=None) -> int:
    out = ctypes.c_int(-1)
    _check(_lib.cpattn_workspace_status(_ptr(workspace), _stream(stream), ctypes.byref(out)),
           "cpattn_workspace_status")
    return out.value


def cpattn_fwd_step(q, k, v, cu_seqlens_q_dev, cu_seqlens_k_dev, num_seqs, mask_mode, step: Step,
                    softmax_scale, out_partial, lse_partial, workspace, stream=None):
    ws, ws_bytes = _workspace(workspace)
    st = _lib.cpattn_fwd_step(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(_tensor(v)),
                              _cu(cu_seqlens_q_dev, "cu_seqlens_q", num_seqs),
                              _cu(cu_seqlens_k_dev, "cu_seqlens_k", num_seqs), num_seqs, mask_mode,
                              ctypes.byref(step), float(softmax_scale), ctypes.byref(_tensor(out_partial)),
                              _f32(lse_partial, "lse_partial", (q.shape[1], q.shape[0])), ws, ws_bytes,
                              _stream(stream))
    _check(st, "cpattn_fwd_step")


def cpattn_fwd_step_noalloc(q, k, v, cu_seqlens_q_dev, cu_seqlens_k_dev, num_seqs, mask_mode, step: Step,
                            softmax_scale, out_partial, lse_partial, stream=None):
    """cpattn_fwd_step with the schedule workspace inside the library (no
    device allocation by the call; see cpattn.h)."""
    st = _lib.cpattn_fwd_step_noalloc(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(_tensor(v)),
                                      _cu(cu_seqlens_q_dev, "cu_seqlens_q", num_seqs),
                                      _cu(cu_seqlens_k_dev, "cu_seqlens_k", num_seqs), num_seqs, mask_mode,
                                      ctypes.byref(step), float(softmax_scale), ctypes.byref(_tensor(out_partial)),
                                      _f32(lse_partial, "lse_partial", (q.shape[1], q.shape[0])), _stream(stream))
    _check(st, "cpattn_fwd_step_noalloc")


def cpattn_merge(out, lse, out_partial, lse_partial, stream=None):
    t, h, d = out_partial.shape
    st = _lib.cpattn_merge(_f32(out, "out", (t, h, d)), _f32(lse, "lse", (h, t)),
                           ctypes.byref(_tensor(out_partial)), _f32(lse_partial, "lse_partial", (h, t)),
                           _stream(stream))
    _check(st, "cpattn_merge")


def cpattn_fill_f32(t, value: float, stream=None):
    """Every element of the contiguous fp32 tensor t set to value (library kernel)."""
    import torch
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise CpattnError(ERR_INVALID_ARG, "cpattn_fill_f32")
    _check(_lib.cpattn_fill_f32(_ptr(t), t.numel(), float(value), _stream(stream)), "cpattn_fill_f32")


def cpattn_bwd_preprocess(out, dout, delta, stream=None):
    t, h, d = dout.shape
    st = _lib.cpattn_bwd_preprocess(_f32(out, "out", (t, h, d)), ctypes.byref(_tensor(dout)),
                                    _f32(delta, "delta", (h, t)), _stream(stream))
    _check(st, "cpattn_bwd_preprocess")


def cpattn_bwd_step(q, k, v, dout, lse, delta, cu_seqlens_q_dev, cu_seqlens_k_dev, num_seqs, mask_mode,
                    step: Step, softmax_scale, dq_accum, dk_accum, dv_accum, workspace, stream=None):
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    ws, ws_bytes = _workspace(workspace)
    st = _lib.cpattn_bwd_step(ctypes.byref(_tensor(q)), ctypes.byref(_tensor(k)), ctypes.byref(_tensor(v)),
                              ctypes.byref(_tensor(dout)), _f32(lse, "lse", (hq, tq)), _f32(delta, "delta", (hq, tq)),
                              _cu(cu_seqlens_q_dev, "cu_seqlens_q", num_seqs),
                              _cu(cu_seqlens_k_dev, "cu_seqlens_k", num_seqs), num_seqs, mask_mode,
                              ctypes.byref(step), float(softmax_scale), _f32(dq_accum, "dq", (tq, hq, d)),
                              _f32(dk_accum, "dk", (tk, hkv, d)), _f32(dv_accum, "dv", (tk, hkv, d)),
                              ws, ws_bytes, _stream(stream))
    _check(st, "cpattn_bwd_step")


# ---------------------------------------------------------------------------
# Dynamic-CP planner (host only)
# ---------------------------------------------------------------------------
def cpattn_dcp_quotas(m, vpp, pp, total):
    """Eq. 1-3 per-microbatch workload quotas of ranks running m[i] microbatches."""
    mm = np.ascontiguousarray(m, dtype=np.int32)
    W = np.zeros(len(mm), np.float64)
    _check(_lib.cpattn_dcp_quotas(mm.ctypes.data, len(mm), vpp, pp, float(total), W.ctypes.data),
           "cpattn_dcp_quotas")
    return W


def cpattn_dcp_plan_batch(lengths, gpus, max_cp, pp, vpp, mem_tokens, work_quad, work_lin, m_min, m_max,
                          knee_radius=-1):
    """Dynamic-CP plan of a global batch.  Returns a dict with m, knee,
    step_time, sample_bucket [n] and the per-microbatch arrays cp, slot, rank,
    tokens, load (length num_buckets), plus times and budget per m."""
    L = np.ascontiguousarray(lengths, dtype=np.int32)
    cap = int(gpus) * int(m_max)
    nm = int(m_max) - int(m_min) + 1
    arr = {"sample_bucket": np.zeros(len(L), np.int32), "cp": np.zeros(cap, np.int32),
           "slot": np.zeros(cap, np.int32), "rank": np.zeros(cap, np.int32), "tokens": np.zeros(cap, np.int64),
           "load": np.zeros(cap, np.float64), "times": np.zeros(max(nm, 0), np.float64),
           "budget": np.zeros(max(nm, 0), np.float64)}
    cfg = DcpConfig(gpus, max_cp, pp, vpp, mem_tokens, work_quad, work_lin, m_min, m_max, knee_radius)
    out = DcpPlan(0, 0, 0, 0.0, arr["sample_bucket"].ctypes.data, arr["cp"].ctypes.data, arr["slot"].ctypes.data,
                  arr["rank"].ctypes.data, arr["tokens"].ctypes.data, arr["load"].ctypes.data,
                  arr["times"].ctypes.data, arr["budget"].ctypes.data, cap)
    _check(_lib.cpattn_dcp_plan_batch(L.ctypes.data, len(L), ctypes.byref(cfg), ctypes.byref(out)),
           "cpattn_dcp_plan_batch")
    nb = out.num_buckets
    res = {"m": out.m, "knee": out.knee, "num_buckets": nb, "step_time": out.step_time,
           "sample_bucket": arr["sample_bucket"], "times": arr["times"], "budget": arr["budget"]}
    for k in ("cp", "slot", "rank", "tokens", "load"):
        res[k] = arr[k][:nb].copy()
    return res
