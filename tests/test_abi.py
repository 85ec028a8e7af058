"""CPU-side checks of the C-ABI library: it loads, exports every symbol the header declares, and
rejects bad arguments on the host (before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_renorm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return moe.load_library()


def test_library_exports_every_declared_function(lib):
    names = moe.header_functions()
    assert "moe_router_topk" in names and "moe_grouped_swiglu_ffn" in names and len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/moe_rocm.h but not exported"
    assert lib.moe_abi_version() == 1


def test_header_is_plain_c():
    with open(os.path.join(ROOT, "include", "moe_rocm.h")) as f:
        src = f.read()
    assert 'extern "C"' in src
    assert "torch" not in re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def test_workspace_size_arithmetic(lib):
    # one int32 per (16 tokens, expert)
    assert moe.moe_permute_workspace_bytes(4096, 8, 128) == 256 * 128 * 4
    assert moe.moe_permute_workspace_bytes(1, 1, 1) == 4
    assert moe.moe_permute_workspace_bytes(257, 2, 3) == 17 * 3 * 4
    assert moe.moe_router_stats_workspace_bytes(4096, 128) == 32 * 128 * 8
    assert moe.moe_permute_workspace_bytes(0, 2, 3) == 0


NULL = None
S = None  # null stream: never reached, validation fails first


def err(lib):
    return lib.moe_last_error().decode()


@pytest.mark.parametrize("args,status,frag", [
    ((NULL, 4, 8, 9, 1, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "k=9"),        # k > E
    ((NULL, 4, 8, 0, 1, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "k=0"),
    ((NULL, 4, 2000, 8, 1, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "E=2000"),  # E > 1024
    ((NULL, 4, 8, 2, 2, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "renorm=2"),
    ((NULL, 4, 8, 2, 1, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "null"),
    ((NULL, -1, 8, 2, 1, NULL, NULL, S), moe.MOE_ERR_INVALID_ARG, "T=-1"),
])
def test_router_topk_rejects(lib, args, status, frag):
    assert lib.moe_router_topk(*args) == status
    assert frag in err(lib)


def test_router_topk_zero_tokens_is_a_no_op(lib):
    assert lib.moe_router_topk(None, 0, 8, 2, 1, None, None, None) == moe.MOE_OK
    assert err(lib) == ""


def test_router_logits_rejects(lib):
    assert lib.moe_router_logits(None, None, 7, 4, 4, 4, None, None) == moe.MOE_ERR_INVALID_ARG
    assert "dtype" in err(lib)
    assert lib.moe_router_logits(None, None, moe.MOE_BF16, 4, 4, 0, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_logits(None, None, moe.MOE_BF16, 4, 4, 4, None, None) == moe.MOE_ERR_INVALID_ARG
    assert "null" in err(lib)


def test_permute_rejects(lib):
    fake = ctypes.c_void_p(16)  # never dereferenced: validation fails before any launch
    base = [fake, moe.MOE_BF16, 64, 32, fake, 2, 8, fake, fake, fake, fake, fake]
    # workspace too small
    assert lib.moe_permute(*base, fake, 3, None) == moe.MOE_ERR_WORKSPACE
    assert "workspace" in err(lib)
    assert lib.moe_permute(*base, None, 1 << 20, None) == moe.MOE_ERR_WORKSPACE
    bad_k = list(base)
    bad_k[5] = 9
    assert lib.moe_permute(*bad_k, fake, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG
    no_counts = list(base)
    no_counts[8] = None
    assert lib.moe_permute(*no_counts, fake, 1 << 20, None) == moe.MOE_ERR_INVALID_ARG


def test_grouped_ffn_rejects(lib):
    fake = ctypes.c_void_p(256)
    # any H, I in either dtype is accepted (bf16 widths that are not multiples of 8 take the generic
    # kernels); with no rows nothing is launched
    args = [fake, fake, fake, moe.MOE_BF16, 0, 36, 20, 4, fake, fake, None, fake, None]
    assert lib.moe_grouped_swiglu_ffn(*args) == moe.MOE_OK
    args[4] = 64
    args[0] = None
    assert lib.moe_grouped_swiglu_ffn(*args) == moe.MOE_ERR_INVALID_ARG           # null
    args[7] = 0
    assert lib.moe_grouped_swiglu_ffn(*args) == moe.MOE_ERR_INVALID_ARG           # E = 0
    args[7], args[5] = 4, 0
    assert lib.moe_grouped_swiglu_ffn(*args) == moe.MOE_ERR_INVALID_ARG           # H = 0


def test_router_logits_bwd_checks(lib):
    fake = ctypes.c_void_p(64)  # never dereferenced
    # nothing to compute, bad dtype, E out of range, null inputs with tokens
    assert lib.moe_router_logits_bwd(fake, fake, fake, moe.MOE_BF16, 4, 8, 4, None, None, None, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert "nothing to compute" in err(lib)
    assert lib.moe_router_logits_bwd(fake, fake, fake, 7, 4, 8, 4, fake, None, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_logits_bwd(fake, fake, fake, moe.MOE_BF16, 4, 8, 0, fake, None, fake, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert lib.moe_router_logits_bwd(None, fake, fake, moe.MOE_BF16, 4, 8, 4, fake, None, fake, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert "null" in err(lib)
    # no tokens and no weight gradient asked for: d_x has no rows, nothing is launched
    assert lib.moe_router_logits_bwd(None, None, None, moe.MOE_BF16, 0, 8, 4, None, None, fake, None) == moe.MOE_OK


def test_combine_rejects(lib):
    assert lib.moe_unpermute_combine(None, moe.MOE_BF16, 4, 8, 33, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(None, moe.MOE_BF16, 4, 8, 2, None, None, None, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_unpermute_combine(None, moe.MOE_BF16, 0, 8, 2, None, None, None, None, None) == moe.MOE_OK


def test_binding_has_no_cpu_path():
    # the product binding never imports the oracle and has no torch-CPU computation of the layer
    src = open(os.path.join(ROOT, "mixture_experts_layer_renorm_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("no torch-CPU", "")
    assert "import numpy" not in src
