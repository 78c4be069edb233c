"""The C-ABI library: it loads, exports every declared entry point, and its host-only checks work
(no GPU: nothing here launches a kernel or allocates device memory)."""
import ctypes
import os
import re
import subprocess

import pytest

import dispatch_fp8_grouped_amd as mm
from inputs import SHAPES

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mega_moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mega_moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(mm.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", mm.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, n
    lib = mm.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_library_is_gfx950_code():
    """The library (built here by build.py) carries a gfx950 code object and no other target."""
    blob = open(mm.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    for other in (b"--gfx942", b"--gfx90a", b"--gfx1100"):
        assert other not in blob


def cfg_of(name, **kw):
    sh = SHAPES[name]
    args = dict(num_shards=sh.num_shards, max_tokens_per_shard=sh.max_tokens_per_shard, hidden=sh.hidden,
                intermediate=sh.intermediate, num_experts=sh.num_experts,
                num_local_experts=sh.num_local_experts, topk=sh.topk, block_m=sh.block_m)
    args.update(kw)
    return mm.make_config(**args)


@pytest.mark.parametrize("name", list(SHAPES))
def test_workspace_bytes_matches_layout_formula(name):
    sh = SHAPES[name]
    n = mm.mega_moe_workspace_bytes(cfg_of(name))
    S, T, H, I, El, K = (sh.num_shards, sh.max_tokens_per_shard, sh.hidden, sh.intermediate,
                         sh.num_local_experts, sh.topk)
    blocks = -(-(S * T * min(K, El)) // sh.block_m) + El
    rows = blocks * sh.block_m
    # the big regions alone: pool, l2 pool, combine buffer, table
    floor = rows * H + rows * I + K * S * T * H * 2 + El * S * T * 4
    assert floor <= n <= floor + rows * (H // 128 + I // 128 + 3) * 4 + 64 * 2 ** 20
    assert n % 256 == 0
    # the flag adds the fp32 GEMM1 output
    n2 = mm.mega_moe_workspace_bytes(cfg_of(name, flags=mm.FLAG_KEEP_GEMM1_OUTPUT))
    assert n2 >= n + rows * 2 * I * 4


def test_block_m_auto_choice():
    # decode: ~32 rows per expert -> 64; prefill: ~1024 -> 128
    lib = mm.lib()
    for name, want in [("decode", 64), ("prefill", 128), ("tiny", 64)]:
        c = cfg_of(name, block_m=0)
        a = mm.mega_moe_workspace_bytes(c)
        b = mm.mega_moe_workspace_bytes(cfg_of(name, block_m=want))
        assert a == b
    assert lib is not None


@pytest.mark.parametrize("field,value", [
    ("num_shards", 0), ("num_shards", 65), ("hidden", 200), ("hidden", 384), ("intermediate", 100),
    ("num_experts", 250), ("num_local_experts", 0), ("topk", 0), ("topk", 65), ("block_m", 96),
    ("local_rank", 8), ("local_rank", -1), ("flags", 0x80), ("max_tokens_per_shard", 0),
])
def test_unsupported_configs_rejected(field, value):
    c = cfg_of("prefill", **{field: value})
    with pytest.raises(mm.MegaMoEError) as ei:
        mm.mega_moe_workspace_bytes(c)
    assert ei.value.code == mm.ERR_UNSUPPORTED


def test_null_arguments_rejected_without_gpu():
    lib = mm.lib()
    c = cfg_of("tiny")
    assert lib.mega_moe_workspace_bytes(None, None) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_workspace_bytes(ctypes.byref(c), None) == mm.ERR_INVALID_ARG
    h = ctypes.c_void_p()
    # null workspace, misaligned workspace, too-small workspace: all rejected before any HIP call
    assert lib.mega_moe_init(ctypes.byref(c), None, 1 << 20, None, ctypes.byref(h)) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_init(ctypes.byref(c), 0x1008, 1 << 30, None, ctypes.byref(h)) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_init(ctypes.byref(c), 0x100000, 16, None, ctypes.byref(h)) == \
        mm.ERR_WORKSPACE_TOO_SMALL
    assert lib.mega_moe_init(None, 0x100000, 16, None, ctypes.byref(h)) == mm.ERR_INVALID_ARG
    tps = (ctypes.c_int32 * 1)(64)
    assert lib.mega_moe_forward(None, tps, *([None] * 11)) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_status(None, None, None) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_query_layout(None, None) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_set_timing(None, 1) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_stage_times(None, None, None) == mm.ERR_INVALID_ARG
    lib.mega_moe_destroy(None)


def test_strerror_texts():
    for code in (mm.OK, mm.ERR_INVALID_ARG, mm.ERR_UNSUPPORTED, mm.ERR_TOO_MANY_TOKENS,
                 mm.ERR_WORKSPACE_TOO_SMALL, mm.ERR_HIP):
        assert mm.mega_moe_strerror(code) and mm.mega_moe_strerror(code) != "unknown error"
    assert mm.mega_moe_strerror(-99) == "unknown error"


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "dispatch_fp8_grouped_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f
                assert "import inputs" not in text, f


def test_shared_expert_config_and_workspace():
    """A shared expert adds one pool segment of ceil(T_max/BM) blocks and one combine plane; it needs the
    own shard to exist and a free lane after the top-k lanes."""
    base = mm.mega_moe_workspace_bytes(cfg_of("decode"))
    sh = SHAPES["decode"]
    n = mm.mega_moe_workspace_bytes(cfg_of("decode", num_shared_experts=1))
    plane = sh.num_shards * sh.max_tokens_per_shard * sh.hidden * 2
    extra_rows = -(-sh.max_tokens_per_shard // sh.block_m) * sh.block_m
    assert n >= base + plane + extra_rows * (sh.hidden + sh.intermediate)
    lib = mm.lib()
    import ctypes
    # 2 shards, 8 ranks' worth of experts: rank 5 is a valid owner but has no own shard among the 2
    two = dict(num_shards=2, max_tokens_per_shard=64, hidden=256, intermediate=128, num_experts=64,
               num_local_experts=8, topk=4, block_m=64)
    out = ctypes.c_uint64(0)
    c = mm.make_config(**two, local_rank=5)
    assert lib.mega_moe_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == mm.OK
    cases = [mm.make_config(**two, local_rank=5, num_shared_experts=1),
             cfg_of("decode", num_shared_experts=2), cfg_of("decode", num_shared_experts=-1),
             cfg_of("decode", num_shared_experts=1, topk=64)]          # no lane left for slot K
    for c in cases:
        assert lib.mega_moe_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == mm.ERR_UNSUPPORTED
    assert lib.mega_moe_workspace_bytes(ctypes.byref(cfg_of("decode", topk=64)), ctypes.byref(out)) == mm.OK


def test_weight_format_config():
    """MXFP4 and BF16 weights are config values (either with or without the one-launch GEMMs); other
    values, and the in-launch pull (arrival-counted fill, routing in the launch) with MXFP4 or BF16
    weights, are rejected."""
    import ctypes
    lib = mm.lib()
    out = ctypes.c_uint64(0)
    for ok in (cfg_of("decode", weight_format=mm.WEIGHTS_MXFP4),
               cfg_of("decode", weight_format=mm.WEIGHTS_MXFP4, flags=mm.FLAG_ONE_GEMM_LAUNCH),
               cfg_of("decode", flags=mm.FLAG_ONE_GEMM_LAUNCH | mm.FLAG_FILL_IN_GEMM1),
               cfg_of("decode", weight_format=mm.WEIGHTS_BF16),
               cfg_of("decode", weight_format=mm.WEIGHTS_BF16, flags=mm.FLAG_ONE_GEMM_LAUNCH)):
        assert lib.mega_moe_workspace_bytes(ctypes.byref(ok), ctypes.byref(out)) == mm.OK
    for c in (cfg_of("decode", weight_format=3), cfg_of("decode", weight_format=-1),
              cfg_of("decode", weight_format=mm.WEIGHTS_MXFP4, flags=mm.FLAG_FILL_IN_GEMM1),
              cfg_of("decode", weight_format=mm.WEIGHTS_MXFP4, flags=mm.FLAG_ROUTE_IN_LAUNCH),
              cfg_of("decode", weight_format=mm.WEIGHTS_BF16, flags=mm.FLAG_FILL_IN_GEMM1),
              cfg_of("decode", weight_format=mm.WEIGHTS_BF16, flags=mm.FLAG_ONE_GEMM_LAUNCH | mm.FLAG_FILL_IN_GEMM1),
              cfg_of("decode", weight_format=mm.WEIGHTS_BF16, flags=mm.FLAG_ROUTE_IN_LAUNCH)):
        assert lib.mega_moe_workspace_bytes(ctypes.byref(c), ctypes.byref(out)) == mm.ERR_UNSUPPORTED


def test_pack_scales_argument_checks():
    """The exponent transform exists for MXFP4 only: an FP8 config, null and misaligned pointers are
    rejected before any device work (no GPU needed)."""
    import ctypes
    lib = mm.lib()
    a = ctypes.c_void_p(4096)
    fp8, mx = cfg_of("decode"), cfg_of("decode", weight_format=mm.WEIGHTS_MXFP4)
    assert lib.mega_moe_pack_scales(ctypes.byref(fp8), a, a, a, a, None) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_pack_scales(ctypes.byref(mx), None, a, a, a, None) == mm.ERR_INVALID_ARG
    assert lib.mega_moe_pack_scales(ctypes.byref(mx), a, ctypes.c_void_p(4098), a, a, None) == mm.ERR_INVALID_ARG


def test_noalloc_host_checks_refuse_before_any_gpu_call():
    """mega_moe_forward_noalloc: a config whose workspace exceeds the static scratch, and the flags whose
    forwards would record memsets or keep test buffers, are refused by host arithmetic alone."""
    lib = mm.lib()
    tps = (ctypes.c_int32 * 8)(*[1] * 8)
    nul = [None] * 11
    big = cfg_of("prefill")
    assert mm.mega_moe_workspace_bytes(big) > mm.NOALLOC_SCRATCH_BYTES
    assert lib.mega_moe_forward_noalloc(ctypes.byref(big), tps, *nul, None) == mm.ERR_SCRATCH_TOO_SMALL
    dec = cfg_of("decode")
    assert mm.mega_moe_workspace_bytes(dec) <= mm.NOALLOC_SCRATCH_BYTES
    for flag in (mm.FLAG_DEBUG_POISON, mm.FLAG_KEEP_GEMM1_OUTPUT):
        c = cfg_of("decode", flags=flag)
        assert lib.mega_moe_forward_noalloc(ctypes.byref(c), tps, *nul, None) == mm.ERR_UNSUPPORTED
    assert lib.mega_moe_forward_noalloc(None, tps, *nul, None) == mm.ERR_INVALID_ARG
    assert "static scratch" in mm.mega_moe_strerror(mm.ERR_SCRATCH_TOO_SMALL)
