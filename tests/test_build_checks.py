"""Host-side checks of the build's scan of generated gfx950 code (no GPU)."""
from linear_attention_state_anchor_amd.build import check_mfma_chains

# A 16x16x32 result accumulated by a 16x16x16 MFMA one wait state later (the
# form that read stale accumulators), the reverse order, and safe forms.
ASM = """\
_ZN2sr1kEv:
\tv_mfma_f32_16x16x32_f16 v[84:87], v[96:99], v[84:87], v[100:103]
\ts_nop 0
\tv_mfma_f32_16x16x16_f16 v[84:87], v[106:107], v[88:89], v[84:87]
\tv_mfma_f32_16x16x16_f16 v[40:43], v[2:3], v[4:5], 0
\tv_add_u32_e32 v9, 1, v9
\tv_mfma_f32_16x16x32_f16 v[40:43], v[8:11], v[12:15], v[40:43]
_ZN2sr2k2Ev:
\tv_mfma_f32_16x16x32_f16 v[0:3], v[8:11], v[12:15], v[0:3]
\tv_mfma_f32_16x16x32_f16 v[0:3], v[16:19], v[12:15], v[0:3]
\tv_mfma_f32_16x16x32_f16 v[20:23], v[8:11], v[12:15], 0
\ts_nop 7
\tv_mfma_f32_16x16x16_f16 v[20:23], v[2:3], v[4:5], v[20:23]
\tv_mfma_f32_16x16x32_f16 v[24:27], v[8:11], v[12:15], 0
\tv_cvt_f32_f16_e32 v24, v1
\tv_mfma_f32_16x16x16_f16 v[24:27], v[2:3], v[4:5], v[24:27]
"""


def test_flags_mixed_shape_accumulation_without_wait_states():
    bad = check_mfma_chains(ASM)
    assert len(bad) == 3, bad
    assert bad[0].startswith("_ZN2sr1kEv:") and "16x16x16_f16 v[84:87]" in bad[0]
    assert "1 wait states earlier" in bad[0]
    assert "16x16x32_f16 v[40:43]" in bad[1] and "16x16x16" in bad[1].split("onto")[1]
    # k2: the same-shape chain and the pair 8 wait states apart pass; a VALU
    # write of one accumulator register leaves the other three in the chain
    assert bad[2].startswith("_ZN2sr2k2Ev:") and "v[24:27]" in bad[2]


def test_threshold_and_intervening_write():
    # the s_nop 7 pair (8 wait states) passes at the default threshold and
    # is flagged when more are demanded; a VALU write to the accumulator
    # between the two MFMAs ends the chain only for the registers it writes
    strict = check_mfma_chains(ASM, min_wait_states=10)
    assert any("v[20:23]" in b for b in strict)
    assert not any("v[20:23]" in b for b in check_mfma_chains(ASM))


def test_clean_code_passes():
    ok = ("k:\n\tv_mfma_f32_16x16x32_f16 v[0:3], v[8:11], v[12:15], v[0:3]\n"
          "\tv_mfma_f32_16x16x32_f16 v[0:3], v[8:11], v[12:15], v[0:3]\n"
          "\tv_cvt_pk_f16_f32 v4, v0, v1\n\tv_cvt_pk_f16_f32 v5, v2, v3\n"
          "\tv_mfma_f32_16x16x16_f16 v[0:3], v[4:5], v[6:7], 0\n")
    assert check_mfma_chains(ok) == []
