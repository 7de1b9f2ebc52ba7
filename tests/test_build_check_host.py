"""Host checks of the build's scan of the generated gfx950 code for a vector
instruction that overwrites the accumulator input of an in-flight
v_mfma_f32_16x16x16_bf16 (``build.srcc_war_hazards``).  The snippets are the
shape of the code that gave wrong results: a weight tile copied into the
accumulator input of the next product four wait states after its issue."""
from test_rnn_layer_ttt_amd.build import SRCC_WAR_MIN, srcc_war_hazards

HAZARD = """
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[62:65], v[54:57], a[0:3]
\tv_mfma_f32_16x16x16_bf16 a[16:19], v[58:59], v[66:67], a[0:3]
\tds_write_b16 v98, v68 offset:62960
\tds_write_b16 v98, v69 offset:60800
\tds_write_b16 v98, v138 offset:63104
\tds_write_b16 v98, v139 offset:60944
\tv_accvgpr_write_b32 a0, v42          ; the next tile, into a0
\tv_accvgpr_write_b32 a1, v43
"""


def test_overwrite_four_wait_states_after_issue_is_found():
    h = srcc_war_hazards(HAZARD)
    assert len(h) == 1
    mfma, writer, ws = h[0]
    assert "16x16x16" in mfma and writer.startswith("v_accvgpr_write_b32 a0") and ws == 4


def test_enough_wait_states_pass():
    spaced = HAZARD.replace("\tv_accvgpr_write_b32 a0", f"\ts_nop {SRCC_WAR_MIN - 5}\n"
                            "\tv_accvgpr_write_b32 a0")
    assert srcc_war_hazards(spaced) == []


def test_in_place_accumulation_and_other_writes_pass():
    in_place = """
\tv_mfma_f32_16x16x16_bf16 a[0:3], v[58:59], v[66:67], a[0:3]
\tv_accvgpr_write_b32 a0, v42
\tv_mfma_f32_16x16x16_bf16 a[4:7], v[58:59], v[66:67], a[0:3]
\tv_mov_b32_e32 v10, v11
\tds_write_b64 v0, v[0:1]
\tglobal_store_dwordx4 v[2:3], v[4:7], off
"""
    # first product accumulates in place (its input is its output); the second
    # reads a[0:3], which nothing overwrites afterwards
    assert srcc_war_hazards(in_place) == []


def test_the_wider_product_is_not_flagged():
    wide = HAZARD.replace("v_mfma_f32_16x16x16_bf16 a[16:19], v[58:59], v[66:67]",
                          "v_mfma_f32_16x16x32_bf16 a[16:19], v[58:61], v[66:69]")
    assert srcc_war_hazards(wide) == []


def test_vgpr_accumulator_inputs_are_tracked():
    vg = """
\tv_mfma_f32_16x16x16_bf16 v[20:23], v[58:59], v[66:67], v[10:13]
\tv_cvt_pk_bf16_f32 v12, v1, v2
"""
    assert len(srcc_war_hazards(vg)) == 1


def test_the_serial_pass_products_are_checked_too():
    # the serial pass's 4x4x1 fp32 products (in-tile updates of the row
    # groups) are held to the same rule: a rotated accumulator whose input
    # register is overwritten at once is found, an in-place one passes
    rotated = """
\tv_mfma_f32_4x4x1_16b_f32 v[138:141], v183, v127, v[224:227]
\tv_add_f32_dpp v224, v236, v236 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1
"""
    h = srcc_war_hazards(rotated)
    assert len(h) == 1 and "4x4x1" in h[0][0] and h[0][2] == 0
    in_place = """
\tv_mfma_f32_4x4x1_16b_f32 v[98:101], v188, v94, v[98:101]
\tv_add_f32_dpp v188, v206, v206 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1
"""
    assert srcc_war_hazards(in_place) == []
