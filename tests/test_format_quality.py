"""Error against bytes of the formats and their variants (CPU, oracle): the orderings that the
quantizers' definitions imply must hold on seeded data of the headline and the 8k workloads."""

import pytest

from format_quality import measure


@pytest.mark.parametrize("workload", ["c2_b64_s32k", "c2_b16_s8k"])
def test_format_error_orderings(workload):
    r = {(x["fmt"], x["outlier"]) + ((x["mask"],) if x["mask"] else ()): x
         for x in measure(workload, slices=2, tokens=512)}
    c2, u2 = r[("c2", "e4m3")], r[("u2", "e4m3")]
    # same storage, same bytes: the variants differ only in the fit
    assert c2["bits_per_element"] == u2["bits_per_element"]
    assert r[("int4", "fp16")]["bits_per_element"] == r[("int4s", "fp16")]["bits_per_element"]
    assert r[("int3", "fp16")]["bits_per_element"] < r[("int4", "fp16")]["bits_per_element"]
    # Lloyd iterations from quartile seeds reduce the squared error of the uniform codebook
    for k in ("k_rel_rmse", "v_rel_rmse"):
        assert c2[k] < u2[k]
        assert r[("c2", "none")][k] < r[("u2", "none")][k]
        # 16 levels beat 4; the asymmetric INT4 grid spans [min, max], the symmetric one
        # [-absmax, absmax] with one level unused on the short side
        assert r[("int4", "fp16")][k] < r[("int4s", "fp16")][k] < c2[k]
        assert r[("fp4", "fp16")][k] < c2[k]
        # 8 levels of the same asymmetric grid: between INT4 and the 2-bit codebook
        assert r[("int4", "fp16")][k] < r[("int3", "fp16")][k] < c2[k]
    # isolating outliers costs bytes and lowers the key error of both 2-bit codebooks
    assert c2["bits_per_element"] > r[("c2", "none")]["bits_per_element"] == 3.0
    assert c2["k_rel_rmse"] < r[("c2", "none")]["k_rel_rmse"]
    assert u2["k_rel_rmse"] < r[("u2", "none")]["k_rel_rmse"]
    # attention through 4-bit caches is closer to the unquantized result than through 2-bit ones
    for f in (("int4", "fp16"), ("int4s", "fp16"), ("fp4", "fp16")):
        assert r[f]["attn_rel_rms"] < c2["attn_rel_rms"] < u2["attn_rel_rms"]


def test_channel_mask_on_scaled_channels():
    # on data whose lists each have 4 channels scaled x20, keeping those 4 channels as fp16
    # records costs 4 x 6 bytes per row and leaves every other channel on the unscaled grid:
    # the INT4 error drops below that of the tau-sigma isolation
    r = {(x["fmt"], x["outlier"], x["mask"]): x for x in measure("int4_b1_s1k", slices=2, tokens=512)}
    masked, tau = r[("int4", "fp16", 4)], r[("int4", "fp16", 0)]
    assert masked["bits_per_element"] > tau["bits_per_element"]
    assert masked["k_rel_rmse"] < tau["k_rel_rmse"] and masked["v_rel_rmse"] < tau["v_rel_rmse"]
    assert masked["attn_rel_rms"] < tau["attn_rel_rms"]
