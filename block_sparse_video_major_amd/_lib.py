"""ctypes binding of libvsa.so, with the same entry-point names as the C ABI.

Argument marshalling only: the functions check that each torch tensor has the
shape, dtype, device and layout the C ABI assumes (the C side cannot see
buffer sizes, so this is what keeps every launch in bounds), then pass raw
device pointers and the current HIP stream.  All arithmetic runs in the HIP
kernels.  There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import collections
import ctypes
import dataclasses
import os
import threading
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvsa.so")

VSA_BF16 = 0
VSA_F32 = 1

VSA_OK = 0
VSA_ERR_NULL = -1
VSA_ERR_SHAPE = -2
VSA_ERR_TOPK = -3
VSA_ERR_UNSUPPORTED = -4
VSA_ERR_HIP = -5
VSA_ERR_LUT = -6
VSA_ERR_WORKSPACE = -7


class VsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({vsa_status_str(status)})")


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "heads", "T", "H", "W", "ct", "ch", "cw", "head_dim", "heads_kv", "cube_order",
                 "head_dim_v")] + \
               [("cube_coords", ctypes.c_void_p)]


VSA_CUBES_RASTER, VSA_CUBES_HILBERT = 0, 1
_CUBE_ORDERS = {"raster": VSA_CUBES_RASTER, "hilbert": VSA_CUBES_HILBERT}
# (grid, cube, order, device) -> device table of packed cube coordinates, for
# the last _TABLE_CACHE_SIZE keys (a table is 4 bytes per cube)
_TABLE_CACHE_SIZE = 16
_tables: "collections.OrderedDict" = collections.OrderedDict()
_tables_lock = threading.Lock()


@dataclasses.dataclass(frozen=True)
class Problem:
    """Token grid T x H x W, cube (ct, ch, cw), heads and head size."""
    batch: int
    heads: int
    T: int
    H: int
    W: int
    ct: int = 4
    ch: int = 4
    cw: int = 4
    head_dim: int = 128
    heads_kv: int = 0          # key/value heads (grouped heads); 0 means heads
    cube_order: str = "raster"   # "raster" or "hilbert": the order of the cubes
    head_dim_v: int = 0        # value head size; 0 means head_dim

    @property
    def n_tokens(self) -> int:
        return self.T * self.H * self.W

    @property
    def cube_volume(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def cube_grid(self) -> tuple:
        """Cubes along t, h, w (a grid that does not divide is padded up)."""
        return (-(-self.T // self.ct), -(-self.H // self.ch), -(-self.W // self.cw))

    @property
    def n_cubes(self) -> int:
        gt, gh, gw = self.cube_grid
        return gt * gh * gw

    @property
    def n_positions(self) -> int:
        """Rows of a cube-major token tensor: n_cubes * cube_volume (N when
        the grid divides into cubes, more when it is padded)."""
        return self.n_cubes * self.cube_volume

    @property
    def padded(self) -> bool:
        return self.n_positions != self.n_tokens

    @property
    def kv_heads(self) -> int:
        return self.heads_kv if self.heads_kv else self.heads

    @property
    def v_dim(self) -> int:
        return self.head_dim_v if self.head_dim_v else self.head_dim

    def kv_problem(self) -> "Problem":
        """The problem of a key tensor alone (for the single-tensor reorders
        and pools); also a value tensor's when the head sizes agree."""
        return dataclasses.replace(self, heads=self.kv_heads, heads_kv=0, head_dim_v=0)

    def v_problem(self) -> "Problem":
        """The problem of a value tensor alone: key/value heads, value head size."""
        return dataclasses.replace(self, heads=self.kv_heads, heads_kv=0, head_dim=self.v_dim, head_dim_v=0)

    def c_struct(self, device=None) -> _Problem:
        """The C struct; with the Hilbert order and a device, cube_coords
        points at that device's copy of vsa_cube_table's table (made once
        per grid and device, then kept)."""
        if self.cube_order not in _CUBE_ORDERS:
            raise ValueError(f"cube_order {self.cube_order!r} is not one of {sorted(_CUBE_ORDERS)}")
        order = _CUBE_ORDERS[self.cube_order]
        st = _Problem(self.batch, self.heads, self.T, self.H, self.W,
                      self.ct, self.ch, self.cw, self.head_dim, self.heads_kv, order, self.head_dim_v, None)
        if order != VSA_CUBES_RASTER and device is not None and torch.device(device).type == "cuda":
            st.cube_coords = _cube_table(self, torch.device(device)).data_ptr()
        return st



_lib = None


def load() -> ctypes.CDLL:
    """Load libvsa.so (built by block_sparse_video_major_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_video_major_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_Problem)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    sigs = {
        "vsa_permute": [P, i32, vp, vp, vp],
        "vsa_unpermute": [P, i32, vp, vp, vp],
        "vsa_pool": [P, i32, vp, vp, vp],
        "vsa_permute_pool": [P, i32, vp, vp, vp, vp],
        "vsa_coarse_topk": [P, i32, vp, vp, vp, vp, vp, vp, vp],
        "vsa_sparse_attn_fwd": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp],
        "vsa_sparse_attn_fwd_raster": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp],
        "vsa_sparse_attn_fwd_gather": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp],
        "vsa_check_lut": [P, vp, vp, i32, vp, vp],
        "vsa_mask_to_lut": [P, vp, i32, vp, vp, vp, vp],
        "vsa_sparse_attn_bwd_workspace_size": [P, i32, ctypes.POINTER(ctypes.c_size_t)],
        "vsa_sparse_attn_bwd": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "vsa_sparse_attn_bwd_noalloc": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp],
        "vsa_combine_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "vsa_combine": [P, vp, vp, vp, vp, vp, vp],
        "vsa_coarse_bwd_workspace_size": [P, ctypes.POINTER(ctypes.c_size_t)],
        "vsa_coarse_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "vsa_pool_unpermute_bwd": [P, vp, vp, vp, vp],
        "vsa_permute_bnhd": [P, i32, vp, vp, vp],
        "vsa_permute_pool_bnhd": [P, i32, vp, vp, vp, vp],
        "vsa_sparse_attn_fwd_bnhd": [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp],
        "vsa_pool_unpermute_bwd_bnhd": [P, vp, vp, vp, vp],
        "vsa_perm_index": [P, vp],
        "vsa_cube_table": [P, vp],
        "vsa_status_str": [ctypes.c_int],
        "vsa_abi_version": [],
        "vsa_device_peak": [i32, vp, vp, vp],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "vsa_status_str" else ctypes.c_int
    _lib = lib
    return lib


def vsa_cube_table(p: "Problem") -> torch.Tensor:
    """Packed grid coordinates (t << 20 | h << 10 | w) of the cubes in p's
    cube order (host int32 tensor of n_cubes)."""
    out = torch.empty(p.n_cubes, dtype=torch.int32)
    _check(load().vsa_cube_table(ctypes.byref(p.c_struct()), out.data_ptr()), "vsa_cube_table")
    return out


def _cube_table(p: "Problem", device: torch.device) -> torch.Tensor:
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    key = (p.T, p.H, p.W, p.ct, p.ch, p.cw, p.cube_order, str(device))
    with _tables_lock:
        t = _tables.get(key)
        if t is not None:
            _tables.move_to_end(key)
            return t
    t = vsa_cube_table(p).to(device)
    torch.cuda.synchronize(device)
    with _tables_lock:
        _tables[key] = t
        while len(_tables) > _TABLE_CACHE_SIZE:
            # kernels already queued may still read the oldest table: let
            # them finish before its memory can be reused
            _, old = _tables.popitem(last=False)
            torch.cuda.synchronize(old.device)
    return t


def clear_cube_tables() -> None:
    """Drop the cached cube-coordinate tables (they are rebuilt on demand)."""
    with _tables_lock:
        for t in _tables.values():
            torch.cuda.synchronize(t.device)
        _tables.clear()


def vsa_status_str(status: int) -> str:
    return load().vsa_status_str(int(status)).decode()


def vsa_abi_version() -> int:
    return int(load().vsa_abi_version())


def vsa_device_peak(device: int = 0) -> Tuple[int, int, float]:
    """(compute units, peak shader clock in kHz, dense bf16 MFMA peak in
    TFLOP/s = CUs x clock x 4096 flop per clock) as HIP reports them."""
    cus, khz, tf = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(load().vsa_device_peak(int(device), ctypes.byref(cus), ctypes.byref(khz), ctypes.byref(tf)),
           "vsa_device_peak")
    return int(cus.value), int(khz.value), float(tf.value)


# ---------------------------------------------------------------- helpers

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, shape, dtype, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(status: int, where: str) -> None:
    if status != VSA_OK:
        raise VsaError(status, where)


def _token_dtype(dtype: int):
    if dtype == VSA_BF16:
        return torch.bfloat16
    if dtype == VSA_F32:
        return torch.float32
    raise ValueError(f"dtype code {dtype} is not VSA_BF16 or VSA_F32")


def _tok_shape(p: Problem, d: Optional[int] = None):
    return (p.batch, p.heads, p.n_tokens, d or p.head_dim)


def _bnhd_shape(p: Problem, d: Optional[int] = None):
    return (p.batch, p.n_tokens, p.heads, d or p.head_dim)


def _pos_shape(p: Problem, d: Optional[int] = None):
    """Cube-major token tensor: Np = n_cubes * vol rows."""
    return (p.batch, p.heads, p.n_positions, d or p.head_dim)


def _kv_pos_shape(p: Problem, d: Optional[int] = None):
    return (p.batch, p.kv_heads, p.n_positions, d or p.head_dim)


def _cube_shape(p: Problem, d: Optional[int] = None):
    return (p.batch, p.heads, p.n_cubes, d or p.head_dim)


def _kv_cube_shape(p: Problem, d: Optional[int] = None):
    return (p.batch, p.kv_heads, p.n_cubes, d or p.head_dim)


# ---------------------------------------------------------------- entry points

def vsa_perm_index(p: Problem) -> torch.Tensor:
    """pi[p] = raster index of cube-major position p, -1 at a padded
    position (host int32 tensor of n_positions)."""
    out = torch.empty(p.n_positions, dtype=torch.int32)
    _check(load().vsa_perm_index(ctypes.byref(p.c_struct()), out.data_ptr()), "vsa_perm_index")
    return out


def vsa_permute(p: Problem, dtype: int, x_raster: torch.Tensor, x_cube: torch.Tensor, stream=None) -> None:
    td = _token_dtype(dtype)
    _need(x_raster, "x_raster", _tok_shape(p), td)
    _need(x_cube, "x_cube", _pos_shape(p), td, x_raster.device)
    _check(load().vsa_permute(ctypes.byref(p.c_struct(x_raster.device)), dtype, _ptr(x_raster), _ptr(x_cube),
                              _stream(stream, x_raster.device)), "vsa_permute")


def vsa_unpermute(p: Problem, dtype: int, x_cube: torch.Tensor, x_raster: torch.Tensor, stream=None) -> None:
    td = _token_dtype(dtype)
    _need(x_cube, "x_cube", _pos_shape(p), td)
    _need(x_raster, "x_raster", _tok_shape(p), td, x_cube.device)
    _check(load().vsa_unpermute(ctypes.byref(p.c_struct(x_cube.device)), dtype, _ptr(x_cube), _ptr(x_raster),
                                _stream(stream, x_cube.device)), "vsa_unpermute")


def vsa_pool(p: Problem, dtype: int, x_cube: torch.Tensor, xc: torch.Tensor, stream=None) -> None:
    _need(x_cube, "x_cube", _pos_shape(p), _token_dtype(dtype))
    _need(xc, "xc", _cube_shape(p), torch.float32, x_cube.device)
    _check(load().vsa_pool(ctypes.byref(p.c_struct(x_cube.device)), dtype, _ptr(x_cube), _ptr(xc),
                           _stream(stream, x_cube.device)), "vsa_pool")


def vsa_permute_pool(p: Problem, dtype: int, x_raster: torch.Tensor, x_cube: Optional[torch.Tensor],
                     xc: torch.Tensor, stream=None) -> None:
    """Reorder into cubes and pool in one pass; with x_cube None only the pool (xc) is written."""
    td = _token_dtype(dtype)
    _need(x_raster, "x_raster", _tok_shape(p), td)
    if x_cube is not None:
        _need(x_cube, "x_cube", _pos_shape(p), td, x_raster.device)
    _need(xc, "xc", _cube_shape(p), torch.float32, x_raster.device)
    _check(load().vsa_permute_pool(ctypes.byref(p.c_struct(x_raster.device)), dtype, _ptr(x_raster), _ptr(x_cube), _ptr(xc),
                                   _stream(stream, x_raster.device)), "vsa_permute_pool")


def vsa_coarse_topk(p: Problem, top_k: int, qc: torch.Tensor, kc: torch.Tensor, vc: Optional[torch.Tensor],
                    kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor, oc: Optional[torch.Tensor],
                    stream=None) -> None:
    dev = qc.device
    _need(qc, "qc", _cube_shape(p), torch.float32)
    _need(kc, "kc", _kv_cube_shape(p), torch.float32, dev)
    if vc is not None:
        _need(vc, "vc", _kv_cube_shape(p, p.v_dim), torch.float32, dev)
    if oc is not None:
        _need(oc, "oc", _cube_shape(p, p.v_dim), torch.float32, dev)
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, top_k), torch.int32, dev)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    _check(load().vsa_coarse_topk(ctypes.byref(p.c_struct(dev)), int(top_k), _ptr(qc), _ptr(kc), _ptr(vc),
                                  _ptr(kv_block_idx), _ptr(valid_block_num), _ptr(oc),
                                  _stream(stream, dev)), "vsa_coarse_topk")


def vsa_sparse_attn_fwd(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                        out: torch.Tensor, oc: Optional[torch.Tensor] = None,
                        gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None, stream=None) -> None:
    _fine(p, q, k, v, kv_block_idx, valid_block_num, out, oc, gate_c, gate_f, lse, stream, False)


def vsa_sparse_attn_fwd_raster(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                               out: torch.Tensor, oc: Optional[torch.Tensor] = None,
                               gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """As vsa_sparse_attn_fwd, with gate_c, gate_f, out and lse in raster token order."""
    _fine(p, q, k, v, kv_block_idx, valid_block_num, out, oc, gate_c, gate_f, lse, stream, True)


def vsa_sparse_attn_fwd_gather(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                               out: torch.Tensor, oc: Optional[torch.Tensor] = None,
                               gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                               lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """As vsa_sparse_attn_fwd_raster with q, k and v in raster order too (the kernel gathers their cubes)."""
    _fine(p, q, k, v, kv_block_idx, valid_block_num, out, oc, gate_c, gate_f, lse, stream, "gather")


def vsa_sparse_attn_fwd_bnhd(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                             out: torch.Tensor, oc: Optional[torch.Tensor] = None,
                             gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """As vsa_sparse_attn_fwd_raster with gate_c, gate_f and out as [batch, N, heads, d]."""
    _fine(p, q, k, v, kv_block_idx, valid_block_num, out, oc, gate_c, gate_f, lse, stream, "bnhd")


def _fine(p, q, k, v, kv_block_idx, valid_block_num, out, oc, gate_c, gate_f, lse, stream, raster):
    dev = q.device
    dv = p.v_dim
    os_ = {"bnhd": _bnhd_shape(p, dv), True: _tok_shape(p, dv), "gather": _tok_shape(p, dv),
           False: _pos_shape(p, dv)}[raster]
    if raster == "gather":   # raster token tensors: [batch, heads(_kv), N, d]
        _need(q, "q", _tok_shape(p), torch.bfloat16, dev)
        _need(k, "k", (p.batch, p.kv_heads, p.n_tokens, p.head_dim), torch.bfloat16, dev)
        _need(v, "v", (p.batch, p.kv_heads, p.n_tokens, dv), torch.bfloat16, dev)
    else:
        _need(q, "q", _pos_shape(p), torch.bfloat16, dev)
        _need(k, "k", _kv_pos_shape(p), torch.bfloat16, dev)
        _need(v, "v", _kv_pos_shape(p, dv), torch.bfloat16, dev)
    _need(out, "out", os_, torch.bfloat16, dev)
    if kv_block_idx.dim() != 4:
        raise ValueError("kv_block_idx must be [batch, heads, Nc, max_kv_blocks]")
    max_kv = kv_block_idx.shape[-1]
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, max_kv), torch.int32, dev)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    if oc is not None:
        _need(oc, "oc", _cube_shape(p, dv), torch.float32, dev)
    for name, t in (("gate_c", gate_c), ("gate_f", gate_f)):
        if t is not None:
            _need(t, name, os_, torch.bfloat16, dev)
    if lse is not None:
        _need(lse, "lse", (p.batch, p.heads, p.n_positions if raster is False else p.n_tokens), torch.float32, dev)
    name = {"bnhd": "vsa_sparse_attn_fwd_bnhd", True: "vsa_sparse_attn_fwd_raster",
            "gather": "vsa_sparse_attn_fwd_gather", False: "vsa_sparse_attn_fwd"}[raster]
    _check(getattr(load(), name)(ctypes.byref(p.c_struct(dev)), _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(kv_block_idx), _ptr(valid_block_num), int(max_kv), _ptr(oc),
                                 _ptr(gate_c), _ptr(gate_f), _ptr(out), _ptr(lse),
                                 _stream(stream, dev)), name)


def vsa_check_lut(p: Problem, kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                  bad_rows: torch.Tensor, stream=None) -> None:
    dev = kv_block_idx.device
    if kv_block_idx.dim() != 4:
        raise ValueError("kv_block_idx must be [batch, heads, Nc, max_kv_blocks]")
    max_kv = kv_block_idx.shape[-1]
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, max_kv), torch.int32)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    _need(bad_rows, "bad_rows", (1,), torch.int32, dev)
    _check(load().vsa_check_lut(ctypes.byref(p.c_struct(dev)), _ptr(kv_block_idx), _ptr(valid_block_num),
                                int(max_kv), _ptr(bad_rows), _stream(stream, dev)), "vsa_check_lut")


def vsa_mask_to_lut(p: Problem, mask: torch.Tensor, kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                    overflow_rows: torch.Tensor, stream=None) -> None:
    """Block relation matrix [B, heads, Nc, Nc] (uint8) -> LUT rows and counts."""
    dev = mask.device
    _need(mask, "mask", (p.batch, p.heads, p.n_cubes, p.n_cubes), torch.uint8)
    if kv_block_idx.dim() != 4:
        raise ValueError("kv_block_idx must be [batch, heads, Nc, max_kv_blocks]")
    max_kv = kv_block_idx.shape[-1]
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, max_kv), torch.int32, dev)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    _need(overflow_rows, "overflow_rows", (1,), torch.int32, dev)
    _check(load().vsa_mask_to_lut(ctypes.byref(p.c_struct(dev)), _ptr(mask), int(max_kv), _ptr(kv_block_idx),
                                  _ptr(valid_block_num), _ptr(overflow_rows), _stream(stream, dev)),
           "vsa_mask_to_lut")


def vsa_sparse_attn_bwd_workspace_size(p: Problem, max_kv_blocks: int) -> int:
    """Bytes of device workspace vsa_sparse_attn_bwd needs."""
    n = ctypes.c_size_t(0)
    _check(load().vsa_sparse_attn_bwd_workspace_size(ctypes.byref(p.c_struct()), int(max_kv_blocks),
                                                       ctypes.byref(n)), "vsa_sparse_attn_bwd_workspace_size")
    return int(n.value)


def vsa_sparse_attn_bwd(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                        o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor,
                        dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                        workspace: torch.Tensor, stream=None) -> None:
    """Gradients of the fine attention (all tensors cube-major; dq, dk, dv float32)."""
    dev = q.device
    ts, ks = _pos_shape(p), _kv_pos_shape(p)
    tv, kv = _pos_shape(p, p.v_dim), _kv_pos_shape(p, p.v_dim)   # O, dO and V, dV are d_v wide
    _need(q, "q", ts, torch.bfloat16, dev)
    for name, t in (("o", o), ("d_o", d_o)):
        _need(t, name, tv, torch.bfloat16, dev)
    _need(k, "k", ks, torch.bfloat16, dev)
    _need(v, "v", kv, torch.bfloat16, dev)
    _need(dq, "dq", ts, torch.float32, dev)
    _need(dk, "dk", ks, torch.float32, dev)
    _need(dv, "dv", kv, torch.float32, dev)
    if kv_block_idx.dim() != 4:
        raise ValueError("kv_block_idx must be [batch, heads, Nc, max_kv_blocks]")
    max_kv = kv_block_idx.shape[-1]
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, max_kv), torch.int32, dev)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    _need(lse, "lse", (p.batch, p.heads, p.n_positions), torch.float32, dev)
    if workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D byte tensor")
    _need(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    _check(load().vsa_sparse_attn_bwd(ctypes.byref(p.c_struct(dev)), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(kv_block_idx), _ptr(valid_block_num), int(max_kv), _ptr(o),
                                      _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                      int(workspace.numel()), _stream(stream, dev)), "vsa_sparse_attn_bwd")


def vsa_sparse_attn_bwd_noalloc(p: Problem, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor,
                                o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor,
                                dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, stream=None) -> None:
    """As vsa_sparse_attn_bwd, with the library's fixed per-GPU workspace
    (VSA_NOALLOC_SCRATCH_BYTES) instead of a caller workspace: nothing is
    allocated.  Calls that overlap in time on one GPU race on that workspace.
    (A Hilbert-order problem builds its cube table once per device here.)"""
    dev = q.device
    ts, ks = _pos_shape(p), _kv_pos_shape(p)
    tv, kv = _pos_shape(p, p.v_dim), _kv_pos_shape(p, p.v_dim)
    _need(q, "q", ts, torch.bfloat16, dev)
    for name, t in (("o", o), ("d_o", d_o)):
        _need(t, name, tv, torch.bfloat16, dev)
    _need(k, "k", ks, torch.bfloat16, dev)
    _need(v, "v", kv, torch.bfloat16, dev)
    _need(dq, "dq", ts, torch.float32, dev)
    _need(dk, "dk", ks, torch.float32, dev)
    _need(dv, "dv", kv, torch.float32, dev)
    if kv_block_idx.dim() != 4:
        raise ValueError("kv_block_idx must be [batch, heads, Nc, max_kv_blocks]")
    max_kv = kv_block_idx.shape[-1]
    _need(kv_block_idx, "kv_block_idx", (p.batch, p.heads, p.n_cubes, max_kv), torch.int32, dev)
    _need(valid_block_num, "valid_block_num", (p.batch, p.heads, p.n_cubes), torch.int32, dev)
    _need(lse, "lse", (p.batch, p.heads, p.n_positions), torch.float32, dev)
    _check(load().vsa_sparse_attn_bwd_noalloc(ctypes.byref(p.c_struct(dev)), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(kv_block_idx), _ptr(valid_block_num), int(max_kv), _ptr(o),
                                              _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(dk), _ptr(dv),
                                              _stream(stream, dev)), "vsa_sparse_attn_bwd_noalloc")


def vsa_combine(p: Problem, o_f: torch.Tensor, out: torch.Tensor, oc: Optional[torch.Tensor] = None,
                gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None, stream=None) -> None:
    """out (raster) = g_f * O_f (cube-major) + g_c * O_c per cube, bf16; a
    missing gate_f reads as 1 and a missing gate_c as 0."""
    dev = o_f.device
    _need(o_f, "o_f", _pos_shape(p, p.v_dim), torch.bfloat16, dev)
    _need(out, "out", _tok_shape(p, p.v_dim), torch.bfloat16, dev)
    for name, t in (("gate_c", gate_c), ("gate_f", gate_f)):
        if t is not None:
            _need(t, name, _tok_shape(p, p.v_dim), torch.bfloat16, dev)
    if oc is not None:
        _need(oc, "oc", _cube_shape(p, p.v_dim), torch.float32, dev)
    _check(load().vsa_combine(ctypes.byref(p.c_struct(dev)), _ptr(o_f), _ptr(oc), _ptr(gate_c), _ptr(gate_f),
                              _ptr(out), _stream(stream, dev)), "vsa_combine")


def vsa_combine_bwd(p: Problem, dout: torch.Tensor, d_of: torch.Tensor, d_oc: torch.Tensor,
                    o_f: Optional[torch.Tensor] = None, oc: Optional[torch.Tensor] = None,
                    gate_c: Optional[torch.Tensor] = None, gate_f: Optional[torch.Tensor] = None,
                    d_gate_c: Optional[torch.Tensor] = None, d_gate_f: Optional[torch.Tensor] = None,
                    stream=None) -> None:
    """Gradients of the gated combination (cube-major token tensors)."""
    dev = dout.device
    ts, cs = _pos_shape(p, p.v_dim), _cube_shape(p, p.v_dim)   # all d_v wide
    for name, t in (("dout", dout), ("d_of", d_of), ("o_f", o_f), ("gate_c", gate_c), ("gate_f", gate_f)):
        if t is not None:
            _need(t, name, ts, torch.bfloat16, dev)
    for name, t in (("d_gate_c", d_gate_c), ("d_gate_f", d_gate_f)):
        if t is not None:
            _need(t, name, ts, torch.float32, dev)
    for name, t in (("oc", oc), ("d_oc", d_oc)):
        if t is not None:
            _need(t, name, cs, torch.float32, dev)
    _check(load().vsa_combine_bwd(ctypes.byref(p.c_struct(dev)), _ptr(dout), _ptr(o_f), _ptr(oc), _ptr(gate_c),
                                  _ptr(gate_f), _ptr(d_of), _ptr(d_oc), _ptr(d_gate_c), _ptr(d_gate_f),
                                  _stream(stream, dev)), "vsa_combine_bwd")


def vsa_coarse_bwd_workspace_size(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load().vsa_coarse_bwd_workspace_size(ctypes.byref(p.c_struct()), ctypes.byref(n)),
           "vsa_coarse_bwd_workspace_size")
    return int(n.value)


def vsa_coarse_bwd(p: Problem, qc: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, oc: torch.Tensor,
                   d_oc: torch.Tensor, dqc: torch.Tensor, dkc: torch.Tensor, dvc: torch.Tensor,
                   workspace: torch.Tensor, stream=None) -> None:
    """Gradients of the coarse attention (float32 cube tensors)."""
    dev = qc.device
    cs, kcs = _cube_shape(p), _kv_cube_shape(p)
    for name, t, shape in (("qc", qc, cs), ("dqc", dqc, cs), ("oc", oc, _cube_shape(p, p.v_dim)),
                           ("d_oc", d_oc, _cube_shape(p, p.v_dim)), ("kc", kc, kcs), ("dkc", dkc, kcs),
                           ("vc", vc, _kv_cube_shape(p, p.v_dim)), ("dvc", dvc, _kv_cube_shape(p, p.v_dim))):
        _need(t, name, shape, torch.float32, dev)
    if workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D byte tensor")
    _need(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    _check(load().vsa_coarse_bwd(ctypes.byref(p.c_struct(dev)), _ptr(qc), _ptr(kc), _ptr(vc), _ptr(oc), _ptr(d_oc),
                                 _ptr(dqc), _ptr(dkc), _ptr(dvc), _ptr(workspace), int(workspace.numel()),
                                 _stream(stream, dev)), "vsa_coarse_bwd")


def vsa_pool_unpermute_bwd(p: Problem, dx_cube: torch.Tensor, dxc: Optional[torch.Tensor], dx_raster: torch.Tensor,
                           stream=None) -> None:
    """dx_raster = unpermute(dx_cube + dxc broadcast over each cube / vol), float32."""
    dev = dx_cube.device
    _need(dx_cube, "dx_cube", _pos_shape(p), torch.float32, dev)
    _need(dx_raster, "dx_raster", _tok_shape(p), torch.float32, dev)
    if dxc is not None:
        _need(dxc, "dxc", _cube_shape(p), torch.float32, dev)
    _check(load().vsa_pool_unpermute_bwd(ctypes.byref(p.c_struct(dev)), _ptr(dx_cube), _ptr(dxc), _ptr(dx_raster),
                                         _stream(stream, dev)), "vsa_pool_unpermute_bwd")


def vsa_permute_bnhd(p: Problem, dtype: int, x_bnhd: torch.Tensor, x_cube: torch.Tensor, stream=None) -> None:
    """vsa_permute reading the model layout [batch, N, heads, d]."""
    td = _token_dtype(dtype)
    _need(x_bnhd, "x_bnhd", _bnhd_shape(p), td)
    _need(x_cube, "x_cube", _pos_shape(p), td, x_bnhd.device)
    _check(load().vsa_permute_bnhd(ctypes.byref(p.c_struct(x_bnhd.device)), dtype, _ptr(x_bnhd), _ptr(x_cube),
                                   _stream(stream, x_bnhd.device)), "vsa_permute_bnhd")


def vsa_permute_pool_bnhd(p: Problem, dtype: int, x_bnhd: torch.Tensor, x_cube: Optional[torch.Tensor],
                          xc: torch.Tensor, stream=None) -> None:
    """vsa_permute_pool reading the model layout [batch, N, heads, d] (x_cube None: pool only)."""
    td = _token_dtype(dtype)
    _need(x_bnhd, "x_bnhd", _bnhd_shape(p), td)
    if x_cube is not None:
        _need(x_cube, "x_cube", _pos_shape(p), td, x_bnhd.device)
    _need(xc, "xc", _cube_shape(p), torch.float32, x_bnhd.device)
    _check(load().vsa_permute_pool_bnhd(ctypes.byref(p.c_struct(x_bnhd.device)), dtype, _ptr(x_bnhd), _ptr(x_cube), _ptr(xc),
                                        _stream(stream, x_bnhd.device)), "vsa_permute_pool_bnhd")


def vsa_pool_unpermute_bwd_bnhd(p: Problem, dx_cube: torch.Tensor, dxc: Optional[torch.Tensor],
                                dx_bnhd: torch.Tensor, stream=None) -> None:
    """vsa_pool_unpermute_bwd writing the model layout [batch, N, heads, d]."""
    dev = dx_cube.device
    _need(dx_cube, "dx_cube", _pos_shape(p), torch.float32, dev)
    _need(dx_bnhd, "dx_bnhd", _bnhd_shape(p), torch.float32, dev)
    if dxc is not None:
        _need(dxc, "dxc", _cube_shape(p), torch.float32, dev)
    _check(load().vsa_pool_unpermute_bwd_bnhd(ctypes.byref(p.c_struct(dev)), _ptr(dx_cube), _ptr(dxc), _ptr(dx_bnhd),
                                              _stream(stream, dev)), "vsa_pool_unpermute_bwd_bnhd")
