"""Python binding of libmegamoe, the fused FP8 MoE layer for one GPU's expert-parallel share (MI355X).

Argument marshalling only: every step of the layer runs in the HIP kernels of libmegamoe.so.  The
functions carry the C names of include/mega_moe.h and take torch tensors (device memory) or plain ints.
If the library is not built, loading it raises: there is no fallback path.

    from dispatch_fp8_grouped_amd import MegaMoE
    moe = MegaMoE(num_shards=8, max_tokens_per_shard=4096, hidden=7168, intermediate=2048,
                  num_experts=256, num_local_experts=32, topk=8, block_m=128)
    w1p, w2p = moe.pack_weights(w1, w2)                 # once: the tiled order the GEMMs stream
    y = moe.forward(tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1p, w1_sf, w2p, w2_sf)

With MXFP4 weights (weight_format=WEIGHTS_MXFP4) the exponents are packed once as well,
s1p, s2p = moe.pack_scales(w1_sf, w2_sf), and passed in place of w1_sf / w2_sf.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmegamoe.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_TOO_MANY_TOKENS = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5
ERR_SCRATCH_TOO_SMALL = -6
NOALLOC_SCRATCH_BYTES = 256 << 20

STATUS_BAD_EXPERT_ID = 0x1
STATUS_SLOT_OVERFLOW = 0x2
STATUS_BAD_LAYOUT = 0x4
STATUS_TIMEOUT = 0x8
STATUS_PLACEMENT = 0x10

FLAG_KEEP_GEMM1_OUTPUT = 0x1
FLAG_FILL_IN_GEMM1 = 0x2
FLAG_DEBUG_FORCE_TIMEOUT = 0x4
FLAG_DEBUG_POISON = 0x8
FLAG_ONE_GEMM_LAUNCH = 0x10
FLAG_DEBUG_ROUTE_LAUNCHES = 0x20
FLAG_ROUTE_IN_LAUNCH = 0x40

WEIGHTS_FP8 = 0
WEIGHTS_MXFP4 = 1
WEIGHTS_BF16 = 2
_WEIGHT_FORMATS = {"fp8": WEIGHTS_FP8, "mxfp4": WEIGHTS_MXFP4, "bf16": WEIGHTS_BF16}

STAGE_ROUTE = 0x1
STAGE_FILL = 0x2
STAGE_GEMM1 = 0x4
STAGE_GEMM2 = 0x8
STAGE_COMBINE = 0x10
STAGE_ALL = 0x1F
NUM_STAGES = 5
STAGE_NAMES = ("route", "fill", "gemm1", "gemm2", "combine")

# Exported symbols of include/mega_moe.h
EXPORTS = ("mega_moe_workspace_bytes", "mega_moe_init", "mega_moe_pack_weights", "mega_moe_pack_scales",
           "mega_moe_forward",
           "mega_moe_forward_stages", "mega_moe_forward_noalloc",
           "mega_moe_query_layout", "mega_moe_status", "mega_moe_set_timing", "mega_moe_stage_times",
           "mega_moe_destroy", "mega_moe_strerror")


class MegaMoEError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {mega_moe_strerror(code)} ({code})")
        self.code = code


class mega_moe_config(ctypes.Structure):
    _fields_ = [("num_shards", ctypes.c_int32), ("max_tokens_per_shard", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("num_local_experts", ctypes.c_int32),
                ("local_rank", ctypes.c_int32), ("topk", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("num_shared_experts", ctypes.c_int32),
                ("weight_format", ctypes.c_int32)]


_LAYOUT_U64 = ("status", "chunk_hist", "chunk_base", "send", "recv", "recv_tot", "pool_off", "block_expert",
               "block_index", "table", "pool_x", "pool_sf", "pool_meta", "pool_dst", "l2_x", "l2_sf", "comb", "gemm1_out",
               "sched", "total")


class mega_moe_layout(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int32), ("route_chunks", ctypes.c_int32),
                ("max_pool_blocks", ctypes.c_int32), ("reserved", ctypes.c_int32)] + \
               [(n, ctypes.c_uint64) for n in _LAYOUT_U64]


_lib = None


def lib():
    """The loaded libmegamoe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               f"`python -m dispatch_fp8_grouped_amd.build` (hipcc, gfx950)")
        # torch ships its own libamdhip64.so.7. Loading torch first makes the library bind to that
        # runtime, so torch's streams and allocations are valid handles inside it. Opened the other
        # way round, the process would hold the system runtime and torch's stream handles would fail.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64
        L.mega_moe_workspace_bytes.argtypes = [ctypes.POINTER(mega_moe_config), ctypes.POINTER(u64)]
        L.mega_moe_init.argtypes = [ctypes.POINTER(mega_moe_config), vp, u64, vp, ctypes.POINTER(vp)]
        L.mega_moe_pack_weights.argtypes = [ctypes.POINTER(mega_moe_config), vp, vp, vp, vp, vp]
        L.mega_moe_pack_scales.argtypes = [ctypes.POINTER(mega_moe_config), vp, vp, vp, vp, vp]
        fwd = [vp, ctypes.POINTER(i32), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.mega_moe_forward.argtypes = fwd
        L.mega_moe_forward_stages.argtypes = [vp, u32] + fwd[1:]
        L.mega_moe_forward_noalloc.argtypes = [ctypes.POINTER(mega_moe_config)] + fwd[1:-1] + [vp, vp]
        L.mega_moe_query_layout.argtypes = [vp, ctypes.POINTER(mega_moe_layout)]
        L.mega_moe_status.argtypes = [vp, vp, ctypes.POINTER(u32)]
        L.mega_moe_set_timing.argtypes = [vp, i32]
        L.mega_moe_stage_times.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.mega_moe_destroy.argtypes = [vp]
        L.mega_moe_destroy.restype = None
        L.mega_moe_strerror.argtypes = [i32]
        L.mega_moe_strerror.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name not in ("mega_moe_destroy", "mega_moe_strerror"):
                getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != OK:
        raise MegaMoEError(rc, what)


def _ptr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_config(num_shards, max_tokens_per_shard, hidden, intermediate, num_experts, num_local_experts,
                topk, block_m=0, local_rank=0, flags=0, num_shared_experts=0,
                weight_format=WEIGHTS_FP8) -> mega_moe_config:
    return mega_moe_config(num_shards, max_tokens_per_shard, hidden, intermediate, num_experts,
                           num_local_experts, local_rank, topk, block_m, flags, num_shared_experts, weight_format)


# --------------------------------------------------------------- the C entry points, same names
def mega_moe_strerror(code: int) -> str:
    return lib().mega_moe_strerror(code).decode()


def mega_moe_workspace_bytes(cfg: mega_moe_config) -> int:
    out = ctypes.c_uint64(0)
    _check(lib().mega_moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)), "mega_moe_workspace_bytes")
    return out.value


def mega_moe_init(cfg: mega_moe_config, workspace, workspace_bytes: Optional[int] = None, stream=None):
    h = ctypes.c_void_p()
    nbytes = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    _check(lib().mega_moe_init(ctypes.byref(cfg), _ptr(workspace), nbytes, _stream(stream), ctypes.byref(h)),
           "mega_moe_init")
    return h


def _tps_array(tokens_per_shard: Sequence[int]):
    arr = (ctypes.c_int32 * len(tokens_per_shard))(*[int(t) for t in tokens_per_shard])
    return arr


def mega_moe_forward_stages(h, stages: int, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf,
                            w2, w2_sf, y, cum_recv_stats=None, stream=None):
    rc = lib().mega_moe_forward_stages(h, stages, _tps_array(tokens_per_shard), _ptr(x), _ptr(x_sf),
                                       _ptr(topk_idx), _ptr(topk_weights), _ptr(w1), _ptr(w1_sf), _ptr(w2),
                                       _ptr(w2_sf), _ptr(y), _ptr(cum_recv_stats), _stream(stream))
    _check(rc, "mega_moe_forward_stages")


def mega_moe_pack_weights(cfg: mega_moe_config, w1, w2, w1_packed, w2_packed, stream=None):
    rc = lib().mega_moe_pack_weights(ctypes.byref(cfg), _ptr(w1), _ptr(w2), _ptr(w1_packed), _ptr(w2_packed),
                                     _stream(stream))
    _check(rc, "mega_moe_pack_weights")


def mega_moe_pack_scales(cfg: mega_moe_config, w1_sf, w2_sf, w1_sf_packed, w2_sf_packed, stream=None):
    rc = lib().mega_moe_pack_scales(ctypes.byref(cfg), _ptr(w1_sf), _ptr(w2_sf), _ptr(w1_sf_packed),
                                    _ptr(w2_sf_packed), _stream(stream))
    _check(rc, "mega_moe_pack_scales")


def mega_moe_forward(h, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y,
                     cum_recv_stats=None, stream=None):
    rc = lib().mega_moe_forward(h, _tps_array(tokens_per_shard), _ptr(x), _ptr(x_sf), _ptr(topk_idx),
                                _ptr(topk_weights), _ptr(w1), _ptr(w1_sf), _ptr(w2), _ptr(w2_sf), _ptr(y),
                                _ptr(cum_recv_stats), _stream(stream))
    _check(rc, "mega_moe_forward")


def mega_moe_forward_noalloc(cfg: mega_moe_config, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf,
                             w2, w2_sf, y, cum_recv_stats=None, device_status=None, stream=None):
    """The layer without a handle or workspace (the library's static per-GPU scratch; see the header)."""
    rc = lib().mega_moe_forward_noalloc(ctypes.byref(cfg), _tps_array(tokens_per_shard), _ptr(x), _ptr(x_sf),
                                        _ptr(topk_idx), _ptr(topk_weights), _ptr(w1), _ptr(w1_sf), _ptr(w2),
                                        _ptr(w2_sf), _ptr(y), _ptr(cum_recv_stats), _ptr(device_status),
                                        _stream(stream))
    _check(rc, "mega_moe_forward_noalloc")


def mega_moe_query_layout(h) -> dict:
    L = mega_moe_layout()
    _check(lib().mega_moe_query_layout(h, ctypes.byref(L)), "mega_moe_query_layout")
    return {name: getattr(L, name) for name, _ in mega_moe_layout._fields_}


def mega_moe_status(h, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _check(lib().mega_moe_status(h, _stream(stream), ctypes.byref(v)), "mega_moe_status")
    return v.value


def mega_moe_set_timing(h, enable: bool):
    _check(lib().mega_moe_set_timing(h, 1 if enable else 0), "mega_moe_set_timing")


def mega_moe_stage_times(h, with_count: bool = False):
    """Mean milliseconds per stage over the forwards timed since mega_moe_set_timing(h, True)."""
    arr = (ctypes.c_float * NUM_STAGES)()
    n = ctypes.c_int32(0)
    _check(lib().mega_moe_stage_times(h, arr, ctypes.byref(n)), "mega_moe_stage_times")
    return (list(arr), n.value) if with_count else list(arr)


def mega_moe_destroy(h):
    if h is not None:
        lib().mega_moe_destroy(h)


# --------------------------------------------------------------- convenience object
class MegaMoE:
    """Owns a workspace tensor and a handle; checks tensor shapes and dtypes before each call."""

    def __init__(self, num_shards, max_tokens_per_shard, hidden, intermediate, num_experts, num_local_experts,
                 topk, block_m=0, local_rank=0, flags=0, num_shared_experts=0, weight_format=WEIGHTS_FP8,
                 device="cuda", stream=None):
        import torch
        self.cfg = make_config(num_shards, max_tokens_per_shard, hidden, intermediate, num_experts,
                               num_local_experts, topk, block_m, local_rank, flags, num_shared_experts, weight_format)
        self.nbytes = mega_moe_workspace_bytes(self.cfg)
        self.workspace = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        self.h = mega_moe_init(self.cfg, self.workspace, self.nbytes, stream)
        self.layout = mega_moe_query_layout(self.h)
        self.block_m = self.layout["block_m"]

    @classmethod
    def from_shape(cls, shape, flags=0, **kw):
        return cls(shape.num_shards, shape.max_tokens_per_shard, shape.hidden, shape.intermediate,
                   shape.num_experts, shape.num_local_experts, shape.topk, shape.block_m, shape.local_rank,
                   flags, getattr(shape, "num_shared_experts", 0),
                   _WEIGHT_FORMATS[getattr(shape, "weight_format", "fp8")], **kw)

    def close(self):
        if self.h is not None:
            mega_moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check_inputs(self, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y):
        import torch
        c = self.cfg
        S, T, H, I, El, K = (c.num_shards, c.max_tokens_per_shard, c.hidden, c.intermediate,
                             c.num_local_experts + c.num_shared_experts, c.topk)
        bf16 = c.weight_format == WEIGHTS_BF16
        want = [("x", x, (S, T, H), torch.bfloat16 if bf16 else torch.uint8)]
        if not bf16:
            want += [("x_sf", x_sf, (S, T, H // 128), torch.float32)]
        want += [("topk_idx", topk_idx, (S, T, K), torch.int64),
                ("topk_weights", topk_weights, (S, T, K), torch.float32),
                ("w1 (packed)", w1, self.packed_shapes()[0], torch.uint8),
                ("w2 (packed)", w2, self.packed_shapes()[1], torch.uint8)]
        if c.weight_format == WEIGHTS_MXFP4:
            s1, s2 = self.packed_scale_shapes()
            want += [("w1_sf (packed)", w1_sf, s1, torch.uint8), ("w2_sf (packed)", w2_sf, s2, torch.uint8)]
        elif bf16:
            if x_sf is not None or w1_sf is not None or w2_sf is not None:
                raise ValueError("BF16 x BF16 takes no scales (x_sf, w1_sf, w2_sf must be None)")
        else:
            want += [("w1_sf", w1_sf, (El, 2 * I // 128, H // 128), torch.float32),
                     ("w2_sf", w2_sf, (El, H // 128, I // 128), torch.float32)]
        want += [("y", y, (S, T, H), torch.bfloat16)]
        for name, t, shape, dtype in want:
            if t is None:
                continue
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{name}: want contiguous cuda {dtype} {shape}, got {t.dtype} "
                                 f"{tuple(t.shape)} on {t.device}")

    def packed_shapes(self):
        """Shapes of the packed W1 and W2 (see mega_moe_pack_weights)."""
        c = self.cfg
        El, H, I = c.num_local_experts + c.num_shared_experts, c.hidden, c.intermediate
        if c.weight_format == WEIGHTS_BF16:                        # 128-byte K chunks of 64 values
            return (El, I // 128, H // 64, 256, 128), (El, H // 256, I // 64, 256, 128)
        rb = 64 if c.weight_format == WEIGHTS_MXFP4 else 128     # bytes per row and 128-value K step
        return (El, I // 128, H // 128, 256, rb), (El, H // 256, I // 128, 256, rb)

    def packed_scale_shapes(self):
        """Shapes of the packed MXFP4 exponents (see mega_moe_pack_scales)."""
        c = self.cfg
        El, H, I = c.num_local_experts + c.num_shared_experts, c.hidden, c.intermediate
        return (El, I // 128, H // 128, 256, 4), (El, H // 256, I // 128, 256, 4)

    def pack_scales(self, w1_sf, w2_sf, stream=None):
        """MXFP4 exponents, uint8 [E_w,2I,H/32] and [E_w,H,I/32] -> new packed tensors (w1_sfp, w2_sfp)."""
        import torch
        c = self.cfg
        El, H, I = c.num_local_experts + c.num_shared_experts, c.hidden, c.intermediate
        for name, t, shape in (("w1_sf", w1_sf, (El, 2 * I, H // 32)), ("w2_sf", w2_sf, (El, H, I // 32))):
            if tuple(t.shape) != shape or t.dtype != torch.uint8 or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{name}: want contiguous cuda uint8 {shape}, got {t.dtype} {tuple(t.shape)}")
        s1, s2 = self.packed_scale_shapes()
        p1 = torch.empty(s1, dtype=torch.uint8, device=w1_sf.device)
        p2 = torch.empty(s2, dtype=torch.uint8, device=w2_sf.device)
        mega_moe_pack_scales(self.cfg, w1_sf, w2_sf, p1, p2, stream)
        return p1, p2

    def pack_weights(self, w1, w2, stream=None):
        """Row-major W1 [E_w,2I,H] and W2 [E_w,H,I] (uint8 e4m3fn, or bfloat16 with BF16 weights; E_w = E_l +
        shared experts, the shared expert last) -> new packed tensors (w1p, w2p)."""
        import torch
        c = self.cfg
        El, H, I = c.num_local_experts + c.num_shared_experts, c.hidden, c.intermediate
        d = 2 if c.weight_format == WEIGHTS_MXFP4 else 1          # two e2m1 codes per byte
        dt = torch.bfloat16 if c.weight_format == WEIGHTS_BF16 else torch.uint8
        for name, t, shape in (("w1", w1, (El, 2 * I, H // d)), ("w2", w2, (El, H, I // d))):
            if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{name}: want contiguous cuda {dt} {shape}, got {t.dtype} {tuple(t.shape)}")
        s1, s2 = self.packed_shapes()
        w1p = torch.empty(s1, dtype=torch.uint8, device=w1.device)
        w2p = torch.empty(s2, dtype=torch.uint8, device=w2.device)
        mega_moe_pack_weights(self.cfg, w1, w2, w1p, w2p, stream)
        return w1p, w2p

    def forward(self, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y=None,
                cum_recv_stats=None, stream=None, stages=STAGE_ALL):
        import torch
        if y is None and stages & STAGE_COMBINE:
            c = self.cfg
            y = torch.empty((c.num_shards, c.max_tokens_per_shard, c.hidden), dtype=torch.bfloat16,
                            device=self.workspace.device)
        self._check_inputs(x, x_sf, topk_idx, topk_weights, w1, w1_sf, w2, w2_sf, y)
        mega_moe_forward_stages(self.h, stages, tokens_per_shard, x, x_sf, topk_idx, topk_weights, w1, w1_sf,
                                w2, w2_sf, y, cum_recv_stats, stream)
        return y

    def __call__(self, inputs: dict, y=None, cum_recv_stats=None, stream=None, stages=STAGE_ALL):
        """Forward on an input dict.  The packed weights are taken from inputs["w1_packed"] /
        inputs["w2_packed"]; when absent they are packed from inputs["w1"] / inputs["w2"] once and stored
        there (the one-time weight transform).  MXFP4 exponents are packed the same way into
        inputs["w1_sf_packed"] / inputs["w2_sf_packed"]."""
        if "w1_packed" not in inputs or "w2_packed" not in inputs:
            inputs["w1_packed"], inputs["w2_packed"] = self.pack_weights(inputs["w1"], inputs["w2"], stream)
        s1, s2 = inputs.get("w1_sf"), inputs.get("w2_sf")
        if self.cfg.weight_format == WEIGHTS_MXFP4:
            if "w1_sf_packed" not in inputs or "w2_sf_packed" not in inputs:
                inputs["w1_sf_packed"], inputs["w2_sf_packed"] = self.pack_scales(s1, s2, stream)
            s1, s2 = inputs["w1_sf_packed"], inputs["w2_sf_packed"]
        return self.forward(inputs["tokens_per_shard"], inputs["x"], inputs.get("x_sf"), inputs["topk_idx"],
                            inputs["topk_weights"], inputs["w1_packed"], s1, inputs["w2_packed"],
                            s2, y, cum_recv_stats, stream, stages)

    def status(self, stream=None) -> int:
        return mega_moe_status(self.h, stream)

    def region(self, name: str, dtype, shape):
        """A tensor view of one workspace region (see mega_moe_layout)."""
        import torch
        off = self.layout[name]
        n = 1
        for d in shape:
            n *= d
        itemsize = torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + n * itemsize].view(dtype).view(*shape)
