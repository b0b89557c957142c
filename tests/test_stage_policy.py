"""Host stage policy (bsattn_stage_*) against the rules the SD.Next commit
page states for the sparse stage (CPU only; no GPU is touched).

 - gates: self attention only, a minimum length (default 8192, 0 = no floor,
   negative reserved), no causal flag, and a token mask only when the backend
   composes it with a block mask (masked_block);
 - no capable backend: warn and stay dense;
 - exclusion list: comma separated, case-insensitive, matched against the
   architecture, pipeline class and denoiser class, resolved once per model;
 - budgets: a precomputed per-step schedule with at most two values;
 - a declined call, and a call served without a layout, are reported once per
   length.
"""
import pytest

import head_masked_attention_amd as hm


def test_default_min_length_is_the_measured_crossover():
    st = hm.Stage()
    assert hm.DEFAULT_MIN_LENGTH == 8192
    assert st.decide(8191)["outcome"] == hm.DECLINE_SHORT
    d = st.decide(8192)
    assert d["outcome"] == hm.STAGE_SPARSE and d["budget"] == pytest.approx(0.3)


def test_zero_min_length_sparsifies_every_length():
    st = hm.Stage(min_length=0)
    for n in (1, 64, 4096):
        assert st.decide(n)["outcome"] == hm.STAGE_SPARSE


def test_negative_min_length_is_reserved():
    with pytest.raises(hm.BsattnError):
        hm.Stage(min_length=-1)


@pytest.mark.parametrize("kw,outcome", [
    (dict(self_attention=False), hm.DECLINE_NOT_SELF),
    (dict(kv_len=77), hm.DECLINE_NOT_SELF),
    (dict(causal=True), hm.DECLINE_CAUSAL),
])
def test_gates(kw, outcome):
    st = hm.Stage(min_length=0)
    q = 16384
    kv = kw.pop("kv_len", None)
    assert st.decide(q, kv, **kw)["outcome"] == outcome


def test_token_mask_needs_a_masked_block_backend():
    served = hm.Stage(min_length=0, backend_masked_block=True).decide(10000, has_token_mask=True)
    assert served["outcome"] == hm.STAGE_SPARSE and served["use_key_mask"]
    declined = hm.Stage(min_length=0, backend_masked_block=False).decide(10000, has_token_mask=True)
    assert declined["outcome"] == hm.DECLINE_TOKEN_MASK and not declined["use_key_mask"]


def test_no_capable_backend_warns_and_stays_dense():
    st = hm.Stage(backend_block_mask=False)
    d = st.decide(20000)
    assert d["outcome"] == hm.DECLINE_NO_BACKEND and d["budget"] == 0.0 and d["first_report"]
    assert "dense" in d["reason"]


def test_disabled():
    assert hm.Stage(enabled=False).decide(20000)["outcome"] == hm.DECLINE_DISABLED


def test_exclusion_list_case_insensitive_on_any_of_three_names():
    st = hm.Stage(min_length=0, exclude=" CosmosTransformer3DModel , other ")
    assert st.decide(9000, denoiser="cosmostransformer3dmodel")["outcome"] == hm.DECLINE_EXCLUDED
    assert st.decide(9000, pipeline="COSMOSTRANSFORMER3DMODEL")["outcome"] == hm.DECLINE_EXCLUDED
    assert st.decide(9000, architecture="Other")["outcome"] == hm.DECLINE_EXCLUDED
    assert st.decide(9000, architecture="sdxl", pipeline="p", denoiser="unet")["outcome"] == hm.STAGE_SPARSE
    # a name that merely contains an entry is not a match
    assert st.decide(9000, denoiser="CosmosTransformer3DModelV2")["outcome"] == hm.STAGE_SPARSE


def test_two_value_schedule():
    st = hm.Stage(min_length=0, n_steps=30, schedule=(0.5, 0.2, 10))
    budgets = [st.decide(4096, step=s)["budget"] for s in range(40)]
    assert budgets[:10] == [0.5] * 10 and budgets[10:] == [0.2] * 30
    assert len(set(budgets)) <= 2


@pytest.mark.parametrize("schedule,n_steps", [((0.5, 0.0, 3), 10), ((0.3, 0.3, 11), 10), ((float("nan"), 0.3, 1), 4)])
def test_schedule_validation(schedule, n_steps):
    with pytest.raises(hm.BsattnError):
        hm.Stage(n_steps=n_steps, schedule=schedule)


def test_declines_and_no_layout_are_reported_once_per_length():
    st = hm.Stage()
    first = st.decide(4096)
    again = st.decide(4096, step=3)
    other_len = st.decide(6000)
    assert first["outcome"] == hm.DECLINE_SHORT and first["first_report"]
    assert not again["first_report"]
    assert other_len["first_report"]
    nl = [st.decide(9000, has_layout=False) for _ in range(3)]
    assert all(d["outcome"] == hm.STAGE_SPARSE and d["note"] == hm.NOTE_NO_LAYOUT for d in nl)
    assert [d["first_report"] for d in nl] == [True, False, False]
    quiet = st.decide(9000)
    assert quiet["note"] == hm.NOTE_NONE and not quiet["first_report"]


def test_negative_lengths_rejected():
    with pytest.raises(hm.BsattnError):
        hm.Stage().decide(-5)
