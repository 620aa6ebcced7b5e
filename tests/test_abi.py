"""C ABI: the library loads without a GPU, exports every symbol rse.h
declares, and its host-only calls (sizes, status names, argument checks)
behave as documented.  No device work is issued here."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rse.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from recommender_sparse_embedding_amd import _lib

    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    from recommender_sparse_embedding_amd import _lib

    names = _declared()
    assert {"idmap_find_or_insert", "embedding_bag_fwd", "embedding_bag_bwd_update", "blocks_grow"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings(lib):
    from recommender_sparse_embedding_amd import _lib

    for code, name in _lib.STATUS.items():
        assert lib.rse_status_str(code).decode() == name
    assert lib.rse_status_str(-99).decode() == "RSE_ERR_UNKNOWN"


def _row_bytes(lib, dim, dt, opt):
    out = ctypes.c_int64()
    rc = lib.rse_blocks_row_bytes(dim, dt, opt, ctypes.byref(out))
    return rc, out.value


def test_row_bytes_and_page_sizing(lib):
    # row = weights + optimizer state, 16-byte aligned
    assert _row_bytes(lib, 128, 0, 1) == (0, 1024)      # click-log: w + Adagrad acc
    assert _row_bytes(lib, 64, 0, 2) == (0, 768)        # w + Adam m, v
    assert _row_bytes(lib, 32, 1, 1) == (0, 192)        # bf16 w + fp32 acc
    assert _row_bytes(lib, 16, 0, 0) == (0, 64)
    assert _row_bytes(lib, 8, 1, 0) == (0, 16)
    # "阿里 RecIS：搜广推训练的背景与难点": 1e9 ids x 64 fp32 ~ 256 GB (weights only)
    assert _row_bytes(lib, 64, 0, 0)[1] * 10**9 == 256 * 10**9
    # the same table with Adam state: 2e8 live rows ~ 153.6 GB, within 288 GB of HBM
    assert _row_bytes(lib, 64, 0, 2)[1] * 2 * 10**8 == 153_600_000_000
    # "DLRM ...", 案例 1: 1e8 x 64 fp32 = 25.6 GB
    assert _row_bytes(lib, 64, 0, 0)[1] * 10**8 == 25_600_000_000
    assert _row_bytes(lib, 3, 0, 0)[0] == -2            # unsupported dim
    assert _row_bytes(lib, 4, 1, 0)[0] == -2            # bf16 needs dim >= 8
    assert _row_bytes(lib, 16, 0, 7)[0] == -1           # bad optimizer


def test_sizes_are_host_only_and_monotone(lib):
    sz = ctypes.c_size_t()
    slots = (ctypes.c_int64 * 2)(100, 9)
    assert lib.rse_idmap_mem_size(2, slots, ctypes.byref(sz)) == 0
    assert sz.value == 256 + 256 + (104 + 16) * 16        # header, 2 dir entries (padded), slots
    assert lib.rse_idmap_mem_size(0, slots, ctypes.byref(sz)) == -1
    assert lib.rse_idmap_mem_size(2000, slots, ctypes.byref(sz)) == -1
    prev = 0
    for n in (0, 1, 4096, 10**6):
        assert lib.rse_idmap_workspace_size(n, ctypes.byref(sz)) == 0
        assert sz.value >= prev
        prev = sz.value
    prev = 0
    for n in (1, 4096, 10**6):
        assert lib.rse_bwd_workspace_size(n, 26, 65536, 128, ctypes.byref(sz)) == 0
        assert sz.value >= 16 * n and sz.value >= prev
        prev = sz.value
    assert lib.rse_bwd_workspace_size(-1, 1, 1, 16, ctypes.byref(sz)) == -1
    assert lib.rse_blocks_meta_size(16, ctypes.byref(sz)) == 0 and sz.value == 512   # 256 + 128, 256-aligned


def test_null_handles_rejected_without_gpu_work(lib):
    assert lib.blocks_grow(None, None, 0, None) == -1
    assert lib.embedding_bag_fwd(None, None, 0, None, 1, 1, 0, None, None) == -1
    assert lib.idmap_find_or_insert(None, None, None, 0, None, 1, 1, 1, None, None, None, 0, None) == -1
    assert lib.embedding_bag_bwd_update(None, None, 0, None, 1, 1, 0, None, None, None, None, 0, None) == -1
    assert lib.embedding_bag_bwd_prepare(None, None, 0, None, 1, 1, None, 0, None, None) == -1
    assert lib.embedding_bag_bwd_apply(None, None, None, 1, 1, 0, None, None, None, None, 0, None) == -1
    assert lib.rse_version() == 100


def test_bwd_plan_layout_matches_header():
    # the Python mirror of rse_bwd_plan must match the C layout: two int64,
    # one uint32, three int32 -> 32 bytes
    from recommender_sparse_embedding_amd._lib import RseBwdPlan

    assert ctypes.sizeof(RseBwdPlan) == 32
    text = open(HEADER).read()
    body = re.search(r"typedef struct rse_bwd_plan \{(.*?)\} rse_bwd_plan;", text, flags=re.S).group(1)
    fields = re.findall(r"^\s*(\w+)\s+(\w+);", body, flags=re.M)
    assert [f for _, f in fields] == [n for n, _ in RseBwdPlan._fields_]


def test_binding_rejects_short_buffers_before_any_call():
    """The find writes one offset per lookup and reads the table bounds at
    t * stride for t <= n_tables: buffers too short for that are refused in
    the binding, before the library is called (so no device work starts)."""
    import torch

    import recommender_sparse_embedding_amd as rse

    ids = torch.zeros(10, dtype=torch.int64)
    bounds = torch.tensor([0, 4, 10], dtype=torch.int64)
    n_new = torch.zeros(1, dtype=torch.int64)
    with pytest.raises(ValueError, match="row_off"):
        rse.idmap_find_or_insert(None, None, ids, bounds, 1, 2, torch.zeros(9, dtype=torch.int64), n_new)
    with pytest.raises(ValueError, match="bounds"):
        rse.idmap_find_or_insert(None, None, ids, bounds, 2, 2, torch.zeros(10, dtype=torch.int64), n_new)
    with pytest.raises(ValueError, match="stride"):
        rse.idmap_find_or_insert(None, None, ids, bounds, 0, 2, torch.zeros(10, dtype=torch.int64), n_new)



def test_feature_programs_validated_on_the_host(lib):
    """rse_features_create rejects programs that break the transform rules
    before it touches device memory (the address passed is never used)."""
    from recommender_sparse_embedding_amd._lib import RseFeatureProgram

    def create(specs, bnd=()):
        progs = (RseFeatureProgram * len(specs))()
        for t, (inp, ops) in enumerate(specs):
            progs[t].input, progs[t].n_ops = inp, len(ops)
            for k, (kind, arg, nb) in enumerate(ops):
                progs[t].ops[k].kind, progs[t].ops[k].arg, progs[t].ops[k].n_boundaries = kind, arg, nb
        b = (ctypes.c_double * max(1, len(bnd)))(*bnd)
        h = ctypes.c_void_p()
        return lib.rse_features_create(ctypes.byref(h), ctypes.c_void_p(1 << 20), 1 << 30, progs, len(specs), b,
                                       len(bnd), None)

    INV = -1
    F64, I64, HASH, MOD, BUCK = 1, 0, 1, 2, 3
    assert create([(F64, [])]) == INV                                  # ends as a float
    assert create([(F64, [(MOD, 3, 0)])]) == INV                       # mod of a float
    assert create([(I64, [(BUCK, 0, 2)])], (0.0, 1.0)) == INV           # bucketize of an int
    assert create([(F64, [(BUCK, 0, 2)])], (1.0, 0.0)) == INV           # descending boundaries
    assert create([(F64, [(BUCK, 1, 2)])], (0.0, 1.0)) == INV           # past the boundary array
    assert create([(F64, [(BUCK, 0, 2)])], (0.0, float("nan"))) == INV  # NaN boundary
    assert create([(I64, [(MOD, 0, 0)])]) == INV                       # modulus 0
    assert create([(I64, [(7, 0, 0)])]) == INV                         # unknown operation
    assert create([(2, [])]) == INV                                    # unknown input kind


def test_new_entry_points_reject_bad_arguments_without_gpu_work(lib):
    """Admission / age / eviction / free list, feature transforms and the
    interaction: null handles and impossible sizes are refused on the host."""
    INV = -1
    sz = ctypes.c_size_t()
    head, cnt = ctypes.c_int64(), ctypes.c_int64()
    assert lib.rse_idmap_set_stamps(None, None, 0) == INV
    assert lib.rse_idmap_set_clock(None, 3) == INV
    assert lib.rse_idmap_set_admission(None, None, 4, 1024, 2, 0, None) == INV
    assert lib.rse_idmap_rehash(None, None, None, 0, None, 0, None) == INV
    assert lib.rse_idmap_rehash_workspace_size(None, None, ctypes.byref(sz)) == INV
    assert lib.rse_blocks_set_free_list(None, None, 0, None) == INV
    assert lib.rse_blocks_free_status(None, ctypes.byref(head), ctypes.byref(cnt), None) == INV
    assert lib.feature_transform(None, None, 0, None, 1, None, None) == INV
    assert lib.rse_features_mem_size(0, 0, ctypes.byref(sz)) == INV
    assert lib.rse_features_mem_size(2, -1, ctypes.byref(sz)) == INV
    assert lib.rse_features_mem_size(2, 10, ctypes.byref(sz)) == 0 and sz.value >= 256 + 2 * 72 + 80
    assert lib.dlrm_interaction_fwd(None, None, -1, 3, 4, None, None) == INV
    assert lib.dlrm_interaction_fwd(None, None, 4, 0, 4, None, None) == INV
    assert lib.dlrm_interaction_bwd(None, None, None, 4, 3, 0, None, None, None) == INV
    # a batch with work but null pointers
    assert lib.dlrm_interaction_fwd(None, None, 4, 3, 4, None, None) == INV
    # 201 fields of dim 128 exceed one sample's LDS: unsupported, not invalid
    assert lib.dlrm_interaction_fwd(None, None, 4, 200, 128, None, None) == -2
