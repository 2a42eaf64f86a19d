"""C ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and validates arguments / plans on the host before any launch."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "si_indexer.h")


@pytest.fixture(scope="module")
def lib():
    from streaming_top_selection_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsi_indexer.so is not built (run __graft_entry__.build())")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(si_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "si_indexer_topk" in names and "si_materialize_topk" in names
    for n in names:
        assert hasattr(lib, n), n
    from streaming_top_selection_amd import _lib
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define SI_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.si_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for st in range(5):
        assert lib.si_status_str(st).decode().startswith("SI_")
    assert b"unknown" in lib.si_status_str(99)


def plan(**kw):
    from streaming_top_selection_amd import api
    args = dict(B=1, S=65536, T=16384, H=64, D=128, m=4, k=512)
    args.update(kw)
    return api.plan(**args)


def test_plan_headline_workload_is_one_chunk_one_partition(lib):
    p = plan()
    assert p.n_chunks == 1 and p.query_chunk == 65536 and p.n_partitions == 1
    # one partition and k <= 512: the lists keep up to 4096 keys and the merge selects
    assert p.key_tile == 512 and p.cand_capacity == 4096
    # candidate keys (4096 slots + 64 pad slots per list) + counts + 16-byte keep rules
    # for every query row, 256-byte aligned parts
    need = 65536 * ((4096 + 64) * 8 + 4 + 16)
    assert need <= p.workspace_bytes < need + 768


def test_plan_million_token_workspace_is_bounded():
    p = plan(S=1048576, T=262144, kc_dtype="e4m3fn")
    assert p.n_chunks * p.query_chunk >= 1048576
    assert p.workspace_bytes <= (3 << 30) + 4096          # auto chunk keeps it <= 3 GiB


def test_plan_small_problems_split_keys_into_partitions():
    p = plan(S=1024, T=256, k=64)
    assert p.n_partitions == 1                             # too few keys to split
    p = plan(B=1, S=8192, T=8192, m=1, k=64)               # 256 query tiles, long rows
    assert p.n_partitions > 1 and p.n_partitions * 64 <= 8192
    assert p.key_partition % p.key_tile == 0


@pytest.mark.parametrize("kt", [64, 512, 768, 1024])
def test_plan_key_tiles(kt):
    p = plan(key_tile=kt)
    assert p.key_tile == kt and p.cand_capacity == 4096
    # the buffer always has room for k kept keys plus one key tile of arrivals
    assert p.cand_capacity - p.key_tile > 512


@pytest.mark.parametrize("kt,cg", [(64, 2048), (512, 2048), (768, 2048), (1024, 2048)])
def test_plan_key_tiles_with_partitions(kt, cg):
    # several key partitions: each list ends cut to its exact top k
    p = plan(S=8192, T=8192, m=1, k=64, key_tile=kt, key_partition=4 * kt)
    assert p.n_partitions > 1
    assert p.key_tile == kt and p.cand_capacity == cg
    assert p.cand_capacity - p.key_tile > 64


def test_plan_large_k_gets_the_large_buffer():
    p = plan(k=2048)
    assert p.cand_capacity == 4096 and p.cand_capacity - p.key_tile > 2048


def test_plan_query_chunk_rounds_up():
    p = plan(query_chunk=1000)
    assert p.query_chunk == 1024 and p.n_chunks == 64


@pytest.mark.parametrize("kw,status", [
    (dict(D=64), "UNSUPPORTED"), (dict(H=129), "UNSUPPORTED"), (dict(k=4096), "UNSUPPORTED"),
    (dict(key_tile=100), "UNSUPPORTED"), (dict(key_tile=512, key_partition=700), "UNSUPPORTED"),
    (dict(S=8192, T=8192, m=1, k=2048, key_tile=512, key_partition=512), "UNSUPPORTED"),
    (dict(k=0), "INVALID_ARG"), (dict(m=0), "INVALID_ARG"), (dict(S=-1), "INVALID_ARG"),
    (dict(H=0), "INVALID_ARG"), (dict(q_pos0=-5), "INVALID_ARG"), (dict(query_chunk=-1), "INVALID_ARG"),
])
def test_plan_rejects(kw, status):
    from streaming_top_selection_amd import SiError
    with pytest.raises(SiError, match=status):
        plan(**kw)


def _topk(lib, q=None, kc=None, w=None, out=None, ws=None, ws_bytes=0, kc_scale=None,
          kc_dtype=1, B=1, S=64, T=16, H=4, D=128, m=4, k=8):
    from streaming_top_selection_amd import _lib
    cfg = _lib.SiConfig(0, 0, 0, 0)
    return lib.si_indexer_topk(q, 1, kc, kc_dtype, kc_scale, w, B, S, T, H, D, m, k, 0,
                               ctypes.byref(cfg), out, out, ws, ws_bytes, None)


def test_entry_points_validate_before_any_launch(lib):
    """Every call here fails validation, so no device is touched (none exists here)."""
    from streaming_top_selection_amd import _lib
    fake = ctypes.c_void_p(0x100000)                      # never dereferenced
    assert _topk(lib) == _lib.SI_ERR_INVALID_ARG          # NULL inputs
    assert b"NULL" in lib.si_last_error()
    assert _topk(lib, q=fake, kc=fake, w=fake, out=None) == _lib.SI_ERR_INVALID_ARG
    assert _topk(lib, q=fake, kc=fake, w=fake, out=fake, ws=None, ws_bytes=0) == \
        _lib.SI_ERR_WORKSPACE
    assert _topk(lib, q=fake, kc=fake, w=fake, out=fake, kc_dtype=2) == _lib.SI_ERR_INVALID_ARG
    assert _topk(lib, q=fake, kc=fake, w=fake, out=fake, kc_dtype=7) == _lib.SI_ERR_UNSUPPORTED
    assert _topk(lib, q=fake, kc=fake, w=fake, out=fake, k=0) == _lib.SI_ERR_INVALID_ARG
    # misaligned q
    assert _topk(lib, q=ctypes.c_void_p(0x100002), kc=fake, w=fake, out=fake,
                 ws=fake, ws_bytes=1 << 30) == _lib.SI_ERR_INVALID_ARG
    # an empty problem is a successful no-op
    assert _topk(lib, S=0, T=0) == _lib.SI_OK


def test_materialize_validates(lib):
    from streaming_top_selection_amd import _lib
    fake = ctypes.c_void_p(0x100000)
    st = lib.si_materialize_scores(fake, 1, fake, 1, None, fake, 1, 64, 16, 4, 128, 4, 0,
                                   60, 10, fake, None)
    assert st == _lib.SI_ERR_INVALID_ARG                   # rows past S
    st = lib.si_materialize_topk(fake, 1, fake, 1, None, fake, 1, 64, 16, 4, 128, 4, 8, 0,
                                 fake, fake, None, 0, 32, None)
    assert st == _lib.SI_ERR_WORKSPACE                     # no score buffer


def test_python_binding_checks_shapes_without_a_device():
    import torch

    import streaming_top_selection_amd as si
    q = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    kc = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        si.indexer_topk(q, kc, torch.zeros((1, 8, 2)), 2, 2)
    with pytest.raises(ValueError, match="shape"):
        si.indexer_topk(q, kc, torch.zeros((1, 8, 3)), 2, 2)
    with pytest.raises(TypeError):
        si.indexer_topk(q, kc.float(), torch.zeros((1, 8, 2)), 2, 2)


@pytest.mark.parametrize("kw", [
    dict(), dict(S=1024, T=256, k=64), dict(B=2, S=8192, T=2048), dict(S=262144, T=65536),
    dict(S=1048576, T=262144), dict(key_tile=64), dict(key_tile=1024, k=2048),
    dict(query_chunk=1000), dict(S=8192, T=8192, m=1, k=64), dict(key_tile=256, key_partition=4096),
    dict(S=0), dict(B=0),
])
def test_workspace_bytes_matches_plan(lib, kw):
    """si_indexer_topk_workspace_bytes is the plan's workspace at q_pos0 = 0."""
    from streaming_top_selection_amd import api
    args = dict(B=1, S=65536, T=16384, H=64, D=128, m=4, k=512)
    args.update(kw)
    assert api.workspace_bytes(**args) == api.plan(**args).workspace_bytes


def test_workspace_bytes_rejects(lib):
    from streaming_top_selection_amd import SiError, api
    with pytest.raises(SiError, match="2048"):
        api.workspace_bytes(1, 1024, 256, k=4096)
    assert b"2048" in lib.si_last_error()
