"""Host-side checks of the build's scan of generated gfx950 code (no GPU)."""
from linear_attention_state_anchor_amd.build import check_transpose_reads

ASM = """\
_ZN2sr1kEv:
\tv_add_u32_e32 v86, s0, v45
\tds_read_b64_tr_b16 v[36:37], v86 offset:27648
\tds_read_b64_tr_b16 v[86:87], v86 offset:34560
\tds_read_b64_tr_b16 v[40:41], v41 offset:16
\tds_read_b64_tr_b16 v[60:61], v45
\tds_read_b64 v[10:11], v10
_ZN2sr2k2Ev:
\tds_read_b64_tr_b8 v[4:5], v4
"""


def test_flags_destination_overlapping_address():
    bad = check_transpose_reads(ASM)
    assert len(bad) == 3
    assert bad[0].startswith("_ZN2sr1kEv:") and "v[86:87], v86" in bad[0]
    assert "v[40:41], v41" in bad[1]
    assert bad[2].startswith("_ZN2sr2k2Ev:")


def test_plain_reads_and_disjoint_registers_pass():
    ok = "k:\n\tds_read_b64_tr_b16 v[2:3], v4\n\tds_read_b64 v[4:5], v4\n"
    assert check_transpose_reads(ok) == []
