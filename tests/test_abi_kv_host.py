"""Host-side argument checks of the KV-cache entry points (include/paged_kv.h).

No GPU: every call here fails its checks and returns before the library
touches the HIP runtime; the pointers passed are fake, 256-byte aligned,
non-overlapping addresses that are never dereferenced."""
import pytest

import paged_gqa_decode_02_amd as pd

CODES = {name: code for code, name in pd.STATUS_NAMES.items()}
BF16 = pd.PD_DTYPE_BF16
GB = 1 << 30


def rope_call(**over):
    T, Hq, Hkv, D, bs, NB, MP = 8, 32, 8, 128, 16, 64, 4096
    a = dict(q=1 * GB, k=2 * GB, v=3 * GB, qs=Hq * D, ks=Hkv * D, vs=Hkv * D, pos=4 * GB,
             slots=5 * GB, table=6 * GB, maxpos=MP, qo=7 * GB, kc=8 * GB, vc=9 * GB, nb=NB,
             T=T, Hq=Hq, Hkv=Hkv, D=D, bs=bs, dtype=BF16)
    a.update(over)
    return pd.lib.rope_paged_kv_write(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"],
                                      a["pos"], a["slots"], a["table"], a["maxpos"], a["qo"],
                                      a["kc"], a["vc"], a["nb"], a["T"], a["Hq"], a["Hkv"],
                                      a["D"], a["bs"], a["dtype"], 0)


ROPE_ERRORS = [
    (dict(dtype=2), "PD_ERR_DTYPE"),
    (dict(T=-1), "PD_ERR_SHAPE"),
    (dict(Hq=0), "PD_ERR_SHAPE"),
    (dict(Hkv=0), "PD_ERR_SHAPE"),
    (dict(Hq=2048), "PD_ERR_SHAPE"),
    (dict(nb=0), "PD_ERR_SHAPE"),
    (dict(maxpos=0), "PD_ERR_SHAPE"),
    (dict(D=0), "PD_ERR_SHAPE"),
    (dict(D=96, qs=32 * 96, ks=8 * 96, vs=8 * 96), "PD_ERR_UNSUPPORTED"),
    (dict(bs=8), "PD_ERR_UNSUPPORTED"),
    (dict(qs=32 * 128 - 8), "PD_ERR_SHAPE"),
    (dict(ks=8 * 128 - 8), "PD_ERR_SHAPE"),
    (dict(vs=0), "PD_ERR_SHAPE"),
    (dict(T=1 << 24), "PD_ERR_SHAPE"),
    (dict(q=0), "PD_ERR_NULL"),
    (dict(k=0), "PD_ERR_NULL"),
    (dict(v=0), "PD_ERR_NULL"),
    (dict(pos=0), "PD_ERR_NULL"),
    (dict(slots=0), "PD_ERR_NULL"),
    (dict(table=0), "PD_ERR_NULL"),
    (dict(qo=0), "PD_ERR_NULL"),
    (dict(kc=0), "PD_ERR_NULL"),
    (dict(vc=0), "PD_ERR_NULL"),
    (dict(q=GB + 8), "PD_ERR_ALIGN"),
    (dict(kc=8 * GB + 4), "PD_ERR_ALIGN"),
    (dict(table=6 * GB + 8), "PD_ERR_ALIGN"),
    (dict(pos=4 * GB + 2), "PD_ERR_ALIGN"),
    (dict(qs=32 * 128 + 4), "PD_ERR_ALIGN"),
    # outputs overlapping inputs or each other
    (dict(qo=1 * GB + 4096), "PD_ERR_ALIAS"),          # q_out inside q, not in place
    (dict(qo=2 * GB), "PD_ERR_ALIAS"),                 # q_out on k
    (dict(kc=3 * GB), "PD_ERR_ALIAS"),                 # k_cache on v
    (dict(vc=8 * GB + 1024), "PD_ERR_ALIAS"),          # v_cache inside k_cache
    (dict(kc=4 * GB), "PD_ERR_ALIAS"),                 # k_cache on positions
    (dict(vc=6 * GB), "PD_ERR_ALIAS"),                 # v_cache on the table
    (dict(qo=9 * GB), "PD_ERR_ALIAS"),                 # q_out on v_cache
    (dict(q=7 * GB, qs=32 * 128 + 8), "PD_ERR_ALIAS"),  # q_out == q with a strided q
]


@pytest.mark.parametrize("over,code", ROPE_ERRORS)
def test_rope_write_argument_errors(over, code):
    assert rope_call(**over) == CODES[code]


def test_rope_write_zero_tokens_is_a_no_op():
    # checked shapes, then nothing to do: no pointer is needed
    assert rope_call(T=0, q=0, k=0, v=0, pos=0, slots=0, table=0, qo=0, kc=0, vc=0) == 0


def test_rope_write_in_place_q_passes_the_alias_check():
    # q_out == q with contiguous rows is allowed; make it fail later, on the
    # null table, so nothing launches
    assert rope_call(qo=1 * GB, table=0) == CODES["PD_ERR_NULL"]
    assert rope_call(qo=1 * GB, pos=4 * GB + 2) == CODES["PD_ERR_ALIGN"]


TABLE_ERRORS = [
    (dict(maxpos=0), "PD_ERR_SHAPE"),
    (dict(dim=0), "PD_ERR_SHAPE"),
    (dict(dim=127), "PD_ERR_SHAPE"),
    (dict(dim=8192), "PD_ERR_SHAPE"),
    (dict(maxpos=1 << 24, dim=256), "PD_ERR_SHAPE"),
    (dict(base=0.0), "PD_ERR_VALUE"),
    (dict(base=-1.0), "PD_ERR_VALUE"),
    (dict(base=float("inf")), "PD_ERR_VALUE"),
    (dict(base=float("nan")), "PD_ERR_VALUE"),
    (dict(table=0), "PD_ERR_NULL"),
    (dict(table=GB + 4), "PD_ERR_ALIGN"),
]


@pytest.mark.parametrize("over,code", TABLE_ERRORS)
def test_rope_table_argument_errors(over, code):
    a = dict(table=GB, maxpos=4096, dim=128, base=1e6)
    a.update(over)
    assert pd.lib.rope_cos_sin_table(a["table"], a["maxpos"], a["dim"], a["base"], 0) == CODES[code]
