"""CPU-side checks of the C ABI (no GPU needed): libmoe.so loads and
exports every function include/moe.h declares, the host-side argument
checks return the documented status codes before anything is enqueued, and
the sizing helpers agree with the oracle's worst-case formulas."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def L():
    from mixture_experts_layer_04_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mixture_experts_layer_04_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("moe_route", "moe_align", "moe_expert_ffn", "moe_layer"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    from mixture_experts_layer_04_amd._lib import SIGNATURES
    for name in declared_functions():
        assert hasattr(L, name), name
        assert name in SIGNATURES, f"binding lacks {name}"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def test_status_strings(L):
    for s in range(5):
        assert L.moe_status_str(s).startswith(b"MOE_")
    assert L.moe_status_str(99) == b"unknown moe_status"


def test_route_argument_checks(L):
    def call(T=4, H=128, E=8, k=2, ng=1, tg=1, scoring=0, ws=FAKE, nbytes=1 << 20, gf=1):
        return L.moe_route(FAKE, FAKE, gf, None, T, H, E, k, ng, tg, scoring, 1, 1.0, FAKE, FAKE, None, ws, nbytes,
                           None)
    assert call(T=-1) == 1
    assert call(gf=2) == 1 and call(gf=-1) == 1  # gate_is_fp32 is 0 (bf16) or 1 (fp32)
    assert call(gf=0, k=9) == 1       # a bf16 gate is checked the same way
    assert call(H=192) == 1           # H not a multiple of 128
    assert call(k=0) == 1
    assert call(k=9) == 1             # k > E
    assert call(E=2000, k=2) == 1     # E > 1024
    assert call(scoring=7) == 1
    assert call(ng=3) == 1            # does not divide E
    assert call(ng=4, tg=1, k=3) == 1  # k > topk_group * E / n_group
    assert call(ng=8, tg=4) == 1      # groups of one expert
    assert call(ws=None) == 1
    assert call(nbytes=16) == 3       # workspace too small
    assert call(T=(1 << 24) + 1) == 1  # T above 2^24
    assert L.moe_route_workspace_size(1, 128, 8) >= 65536  # control block first
    assert call(T=0) == 0             # empty batch is a no-op


def test_align_argument_checks(L):
    def call(T=4, k=2, E=8, bm=16, ws=FAKE, nbytes=256):
        return L.moe_align(FAKE, T, k, E, bm, FAKE, FAKE, FAKE, ws, nbytes, None)
    assert call(bm=0) == 1
    assert call(bm=2048) == 1
    assert call(E=0) == 1
    assert call(k=17) == 1
    assert call(ws=None) == 1
    assert call(nbytes=4) == 3


def test_route_align_argument_checks(L):
    def call(T=4, H=128, E=8, k=2, bm=16, ws=FAKE, nbytes=1 << 22, ns=0, gf=1):
        return L.moe_route_align(FAKE, FAKE, gf, None, T, H, E, k, ns, 1, 1, 0, 1, 1.0, bm, FAKE, FAKE, FAKE, FAKE,
                                 FAKE, ws, nbytes, None)
    assert call(H=192) == 1           # router checks
    assert call(gf=3) == 1
    assert call(k=9) == 1
    assert call(bm=0) == 1            # alignment checks
    assert call(bm=2048) == 1
    assert call(ws=None) == 1
    assert call(nbytes=16) == 3
    assert call(ns=2) == 1            # at most one shared expert
    assert call(E=1024, ns=1) == 1    # E + n_shared <= 1024
    assert call(k=16, E=32, ns=1) == 1  # k + n_shared <= 16
    need = L.moe_route_align_workspace_size(4096, 2048, 128, 8, 0)
    assert need >= L.moe_route_workspace_size(4096, 2048, 128) and need >= L.moe_align_workspace_size(4096, 8, 128)


def test_ffn_and_layer_argument_checks(L):
    def ffn(T=4, H=256, E=8, F=128, k=2, bm=16, wf=0, ws=FAKE, nbytes=1 << 30, s13=FAKE, lim=math.inf):
        return L.moe_expert_ffn(FAKE, wf, FAKE, s13, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                T, H, E, F, k, bm, lim, FAKE, ws, nbytes, None)
    assert ffn(H=200) == 1            # H not a multiple of 128
    assert ffn(F=96) == 1
    assert ffn(bm=8) == 1             # GEMM blocks are 16, 32, 64 or 128
    assert ffn(wf=5) == 1
    assert ffn(wf=1, s13=None) == 1   # fp8 needs scales
    assert ffn(nbytes=100) == 3
    assert ffn(lim=0.0) == 1 and ffn(lim=-1.0) == 1 and ffn(lim=math.nan) == 1  # SwiGLU limit
    assert ffn(T=0) == 0
    # 32-bit byte offsets: x of 300000 x 7168 bf16 and one expert's w13 of
    # 2 x 32768 x 32768 bf16 are 4 GiB or more
    assert ffn(T=300000, H=7168, F=2048, E=256, k=8, bm=128) == 2
    assert ffn(T=4, H=32768, F=32768) == 2

    def layer(T=4, H=256, E=8, F=128, k=2, bm=0, ws=FAKE, nbytes=1 << 30, ns=0, gf=1):
        return L.moe_layer(FAKE, FAKE, gf, None, 0, FAKE, None, FAKE, None, T, H, E, F, k, ns, 1, 1, 0, 1, 1.0, bm,
                           math.inf, FAKE, None, None, ws, nbytes, None)
    assert layer(bm=48) == 1
    assert layer(gf=2) == 1
    assert layer(ns=2) == 1 and layer(ns=-1) == 1
    assert layer(nbytes=1000) == 3
    assert layer(T=0) == 0


def test_sizing_matches_oracle(L):
    from oracle import align as oalign
    for T, k, E, bm in [(64, 8, 256, 16), (4096, 8, 128, 64), (1, 8, 288, 128), (0, 2, 8, 16)]:
        assert L.moe_align_max_padded(T, k, E, bm) == oalign.max_padded(T * k, E, bm)
        assert L.moe_align_max_blocks(T, k, E, bm) == oalign.max_blocks(T * k, E, bm)


def test_block_m_choice(L):
    # tile height follows the tokens per expert ([Kernels] "The fused expert
    # GEMM", last paragraph): small at decode, large at prefill
    bf16, fp8, mx = 0, 1, 2
    # (T, E, F, k, wformat): from 2 rows per expert on, by rows per expert
    assert L.moe_layer_block_m(64, 256, 2048, 8, fp8) == 32
    assert L.moe_layer_block_m(4096, 128, 768, 8, bf16) == 128
    assert L.moe_layer_block_m(2048, 256, 2048, 8, fp8) == 128  # m = 64: fp8 turns to 128 rows above 44
    assert L.moe_layer_block_m(1536, 256, 2048, 8, fp8) == 128  # m = 48
    assert L.moe_layer_block_m(1280, 256, 2048, 8, fp8) == 64   # m = 40
    assert L.moe_layer_block_m(2048, 256, 2048, 8, bf16) == 64  # m = 64: the others at 96
    assert L.moe_layer_block_m(384, 128, 768, 8, bf16) == 32   # m = 24
    assert L.moe_layer_block_m(448, 128, 768, 8, bf16) == 64   # m = 28
    # below 2: fp8 streams; bf16 / MX by the expected 32-row GEMM1 tiles
    assert L.moe_layer_block_m(63, 256, 2048, 8, fp8) == 16
    assert L.moe_layer_block_m(1, 128, 768, 8, bf16) == 16     # 8 experts x 6 tiles
    assert L.moe_layer_block_m(8, 128, 768, 8, bf16) == 16     # ~51 x 6 = 308 tiles
    assert L.moe_layer_block_m(16, 128, 768, 8, bf16) == 32    # ~81 x 6 = 486 tiles
    assert L.moe_layer_block_m(8, 288, 2304, 8, bf16) == 32    # ~61 x 18 tiles
    assert L.moe_layer_block_m(1, 288, 2304, 8, bf16) == 16
    assert L.moe_layer_block_m(4, 256, 2048, 6, mx) == 32      # ~24 x 16 = 377 tiles
    assert L.moe_layer_block_m(1, 32, 2048, 6, mx) == 16       # 6 x 16 tiles
    assert L.moe_layer_block_m(4, 32, 2048, 6, mx) == 16       # ~18 x 16 = 290 tiles


def test_library_is_built_from_these_sources(L):
    """The library reports the hash of the sources it was built from, and the
    loader refuses one whose hash differs from the sources beside it."""
    from mixture_experts_layer_04_amd import _lib
    assert L.moe_source_hash().decode() == _lib.source_hash()
    saved, real = _lib._lib, _lib.source_hash
    try:
        _lib._lib = None
        _lib.source_hash = lambda: "0000000000000000"
        with pytest.raises(RuntimeError, match="built from other sources"):
            _lib.lib()
    finally:
        _lib._lib, _lib.source_hash = saved, real
