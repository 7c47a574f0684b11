"""Every kernel the library instantiates runs without scratch memory (CPU only: device
compile with the compiler's kernel-resource-usage remarks, nothing is run).

A kernel that spills vector registers to scratch adds per-lane memory traffic to a
path that is bound by HBM bandwidth; SGPR spills go to VGPR lanes and cost no memory
traffic, so only ScratchSize and VGPR spills are held to zero.
"""
import pytest

from paged_kv_decode_blocks_amd.build import SOURCES, kernel_resource_usage


@pytest.fixture(scope="module")
def usage():
    return kernel_resource_usage()


def test_every_hip_source_reports_kernels(usage):
    srcs = {v["source"] for v in usage.values()}
    assert {s for s in SOURCES if s.endswith(".hip")} <= srcs
    assert len(usage) > 100


def test_no_kernel_uses_scratch(usage):
    bad = {k: (v.get("ScratchSize"), v.get("VGPRs Spill")) for k, v in usage.items()
           if v.get("ScratchSize", -1) != 0 or v.get("VGPRs Spill", -1) != 0}
    assert not bad, "kernels with scratch: " + "; ".join(f"{k} {v}" for k, v in sorted(bad.items()))


def test_headline_kernels_keep_their_occupancy(usage):
    """The kernels the workloads' steps run, at the waves per SIMD their launch shapes were
    measured with (registers and LDS both counted by the compiler)."""
    want = {
        "void pkv::decode_mha_kernel<1, 128, 4, 2, 1, true>(pkv::AttnArgs)": 4,     # c2
        "void pkv::decode_mha_kernel<1, 128, 8, 2, 2, true>(pkv::AttnArgs)": 2,     # c3
        "void pkv::decode_mha_kernel<2, 128, 4, 2, 1, true>(pkv::AttnArgs)": 3,     # c4
        "void pkv::decode_gqa_kernel<2, 128, 4, 1, 1, true, true>(pkv::AttnArgs)": 2,   # c5
        "void pkv::decode_fp8_kernel<1, 128, 4, 2, 1, true>(pkv::AttnArgs)": 3,         # c3f8
        "void pkv::decode_gqa_fp8_kernel<2, 128, 4, 1, 1, 2, true>(pkv::AttnArgs)": 3,  # c5f8
        "void pkv::decode_mxfp4_kernel<1, 128, 4, 2>(pkv::AttnArgs)": 3,                # c3f4 attention
        # c5f4: the even split with its one-chunk ring staged through registers (209 VGPRs of 256)
        "void pkv::decode_mxfp4_mfma_kernel<2, 128, 4, 1, true, true, 4, true>(pkv::AttnArgs)": 2,
    }
    for k, occ in want.items():
        assert k in usage, k
        assert usage[k]["Occupancy"] >= occ, (k, usage[k])


def test_tile_read_probe_occupancy(usage):
    """The read probe's waves per SIMD for the grouped kernels' patterns, as the compiler counts
    them (4 items in flight per wave: an LDS ring for the DMA paths, registers for the rest): the resident
    waves per CU are 4x these, which caps what a larger grid adds."""
    want = {
        (1024, 0): 8,    # MXFP4 codes and scales into registers
        (1024, 7): 4,    # MXFP4 codes and scales by DMA: 34 KiB of LDS per workgroup
        (2048, 1): 5,    # FP8: K by DMA (32 KiB), V and scales into registers
        (4096, 0): 3,    # bf16 into registers
        (4096, 1): 2,    # bf16, K by DMA (64 KiB)
    }
    for (tile, paths), occ in want.items():
        for team in (1, 2, 4):
            k = f"void pkv::tile_read_kernel<{tile}, {paths}, {team}, 4>(pkv::TileReadArgs)"
            assert k in usage, k
            assert usage[k]["Occupancy"] == occ, (k, usage[k])
