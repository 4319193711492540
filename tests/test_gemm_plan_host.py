"""Host checks of the GEMM launch planner (knapspec_gemm_plan, no GPU): for the item GEMMs of
every preset shape, the LM-head chunks and odd sizes, at row counts from 1 to 4000, the plan
covers K, the output columns and the rows exactly once, never splits a SwiGLU GEMM, keeps the
partial sums within the room the model reserves, and sends exactly the bf16 K-split
projections with 65..256 rows to the register-activation kernel."""
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ks():
    lib = os.path.join(ROOT, "draft_layer_selection_amd", "libknapspec.so")
    if not os.path.exists(lib):
        from draft_layer_selection_amd import build

        build.build()
    from draft_layer_selection_amd import knapspec

    return knapspec


ROWS = [1, 2, 31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 200, 245, 255, 256, 257, 500, 1024,
        4000]
# (name, n_cols, k, swiglu, d_ff, bf16)
SHAPES = [
    ("tiny qkv", 768, 256, False, 0, False), ("tiny o", 256, 256, False, 0, False),
    ("tiny gate|up", 1536, 256, True, 768, False), ("tiny down", 256, 768, False, 0, False),
    ("f32 d=260", 260, 260, False, 0, False),
    ("qwen qkv", 4096, 2048, False, 0, True), ("qwen o", 2048, 2048, False, 0, True),
    ("qwen gate|up", 12288, 2048, True, 6144, True), ("qwen down", 2048, 6144, False, 0, True),
    ("llama8b qkv", 6144, 4096, False, 0, True), ("llama8b o", 4096, 4096, False, 0, True),
    ("llama8b gate|up", 28672, 4096, True, 14336, True),
    ("llama8b down", 4096, 14336, False, 0, True),
    ("llama70b qkv", 10240, 8192, False, 0, True), ("llama70b o", 8192, 8192, False, 0, True),
    ("llama70b gate|up", 57344, 8192, True, 28672, True),
    ("llama70b down", 8192, 28672, False, 0, True),
    ("lm head chunk", 32768, 4096, False, 0, True), ("lm head last chunk", 4160, 4096, False, 0, True),
    ("f32 lm head ragged", 1000, 256, False, 0, False), ("bf16 dh64 qkv", 3072, 2048, False, 0, True),
]
MAX_SPLITS = 16


def room(rows, n_cols):
    # the model's partial-sum workspace: max(16 * min(R, 256), R) rows of the widest output
    return max(16 * min(rows, 256), rows) * n_cols


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_plan_covers_k_columns_rows(ks, shape):
    _, n, k, swiglu, ff, bf16 = shape
    areg_env = os.environ.get("KNAPSPEC_GEMM_AREG")
    for r in ROWS:
        cap = room(r, n)
        p = ks.gemm_plan(r, n, k, swiglu, ff, bf16, cap)
        what = f"{shape[0]} R={r}: {p}"
        kstep = 64 if bf16 else 32
        # K: splits of k_chunk cover K, the last split non-empty
        assert 1 <= p["splits"] <= MAX_SPLITS, what
        assert p["k_chunk"] > 0 and p["k_chunk"] % kstep == 0, what
        assert (p["splits"] - 1) * p["k_chunk"] < k <= p["splits"] * p["k_chunk"], what
        if swiglu:
            assert p["splits"] == 1, what
        elif p["splits"] > 1:
            assert p["splits"] * r * n <= cap, what
        # routing of the register-activation kernel (default depth 3)
        wants_areg = (bf16 and not swiglu and k % 64 == 0 and n % 128 == 0 and 64 < r <= 256)
        if areg_env is None:
            assert (p["areg"] == 3) == wants_areg, what
        if p["areg"]:
            assert p["ng"] == 0 and p["m_tiles"] == 1 and r <= 256, what
            assert p["n_tiles"] * 128 == n, what
            kiters = (k + 63) // 64
            assert p["splits"] == 1 or p["splits"] <= kiters // (2 * (p["areg"] + 1)), what
            continue
        # columns: every output column in exactly one tile
        if not bf16:
            assert p["n_tiles"] == ((ff + 31) // 32 if swiglu else (n + 63) // 64), what
        elif p["ng"]:
            if swiglu:
                assert p["n_tiles"] * 32 * p["ng"] == ff, what
            else:
                assert p["n_tiles"] * 64 * p["ng"] == n, what
        else:
            assert p["n_tiles"] * (32 if swiglu else 64) == (ff if swiglu else n), what
        # rows: the m-tiles cover every row
        assert p["m_tiles"] * 32 * p["mb"] >= r, what
        assert (p["m_tiles"] - 1) * 32 * p["mb"] < r, what


def test_plan_rejects_bad_arguments(ks):
    with pytest.raises(ks.KnapSpecError):
        ks.gemm_plan(0, 4096, 4096)
    with pytest.raises(ks.KnapSpecError):
        ks.gemm_plan(10, 4096, 4096, swiglu=True, d_ff=1000)  # n_cols != 2 * d_ff
    with pytest.raises(ks.KnapSpecError):
        ks.gemm_plan(10, 1000, 4096)  # bf16 columns not a multiple of 64
    with pytest.raises(ks.KnapSpecError):
        ks.gemm_plan(10, 4096, 4000)  # bf16 K not a multiple of 64
