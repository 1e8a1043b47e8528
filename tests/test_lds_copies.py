"""Every copy of a codebook table into LDS stays in bounds (CPU only).

The kernels copy their lookup tables from the codebook's device allocation
into LDS, some with global_load_lds, one entry per lane.  The library
reports each copy (octo_debug_lds_copy) from the same compile-time constants
its copy loop uses; here every record is checked against the LDS array it
writes and against the entry count of the table it reads, in a codebook of
the record's (d, b, QJL) built host-only: the copy writes no slot past its
LDS array and reads no entry past its table, and a copy whose width does not
divide its slot count bounds each lane.
"""
import functools

import pytest

import rotation_preconditioned_quantization_amd as octo


@pytest.fixture(scope="module")
def records():
    try:
        octo.lib()
    except RuntimeError as e:  # pragma: no cover
        pytest.skip(str(e))
    return octo.octo_debug_lds_copies()


@functools.lru_cache(maxsize=None)
def host_cb(d, b, qjl):
    return octo.Codebook(d, b, qjl=bool(qjl), mc_vectors=4096, device=None)


def test_every_kernel_family_reports_its_copies(records):
    kernels = {r["kernel"] for r in records}
    for k in ("k_logits", "k_attn", "k_mq_attn", "k_encode", "k_encode (joint)", "k_encode (qjl)",
              "k_encode (qjl, joint)", "k_encode_one", "k_encode256", "k_encode256 (joint)"):
        assert k in kernels, k
    shapes = {(r["kernel"], r["d"], r["b"], r["qjl"]) for r in records}
    for d in (64, 128, 256):
        for b in range(1, 6):
            assert ("k_attn", d, b, 0) in shapes and ("k_logits", d, b, 0) in shapes
            if d < 256:
                assert ("k_attn", d, b, 1) in shapes and ("k_logits", d, b, 1) in shapes


def test_copies_stay_in_bounds(records):
    bad = []
    for r in records:
        cb = host_cb(r["d"], r["b"], r["qjl"])
        have = cb.table_entries(r["table"])
        tab = octo.TABLES[r["table"]]
        where = f'{r["kernel"]} d={r["d"]} b={r["b"]} qjl={r["qjl"]} table={tab}'
        if r["slots_written"] > r["lds_slots"]:
            bad.append(f"{where}: writes {r['slots_written']} of {r['lds_slots']} LDS slots")
        if r["entries_read"] == -1:
            if have > r["lds_slots"]:
                bad.append(f"{where}: a {have}-entry table into {r['lds_slots']} LDS slots")
        elif r["entries_read"] > have:
            bad.append(f"{where}: reads {r['entries_read']} entries of a {have}-entry table")
        if not r["masked"] and r["copied"] % r["threads"]:
            bad.append(f"{where}: unmasked copy of {r['copied']} entries by {r['threads']} threads")
        assert have > 0, f"{where}: the codebook has no such table"
    assert not bad, "\n".join(bad)


def test_narrow_copies_are_masked_and_replicas_read_the_whole_table(records):
    """The rho tables (at most 16 entries) are narrower than the threads that
    copy them: only a per-lane bound keeps the other lanes from reading past
    the table.  The replicated code tables (one bit: 16 entries in 16 copies
    fill exactly the 256 slots of k_attn) read every entry and no more."""
    rho = [r for r in records if octo.TABLES[r["table"]] == "rho"]
    assert rho and all(r["masked"] for r in rho if r["copied"] < r["threads"])
    rep = [r for r in records if r["kernel"] == "k_attn" and r["b"] <= 2 and r["d"] == 128
           and octo.TABLES[r["table"]] == "trip"]
    assert rep
    for r in rep:
        assert r["slots_written"] == r["lds_slots"] == r["copied"]
        assert r["entries_read"] == host_cb(r["d"], r["b"], r["qjl"]).table_entries(r["table"])


def test_table_entries_bad_argument():
    cb = host_cb(128, 3, 0)
    assert cb.table_entries(7) == -1 and cb.table_entries(-1) == -1
    assert cb.table_entries(octo.TABLES.index("trip")) == 1024     # 10 bits per triplet at b = 3
    assert cb.table_entries(octo.TABLES.index("s16")) == 0          # no QJL matrix
