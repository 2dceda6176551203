"""The matrix-core pipeline waits of the expert kernels, checked on their
gfx950 assembly (CPU only: hipcc cross-compiles).  The 128-row GEMM blocks
issue MFMAs through inline assembly, for which the compiler inserts no waits;
the audit also runs on the compiler's own MFMA kernels, which must pass it."""
from nvfp4_weight_only_moe_amd import _asm_audit as A


def test_audit_flags_planted_hazards():
    # a VALU write of an MFMA operand right before it, and an MFMA result
    # read at once: both reported; with enough wait states, neither
    bad = """_Zk:
\tv_mul_f32_e32 v4, v1, v2
\tv_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]
\tv_accvgpr_read_b32 v20, a1
\ts_endpgm
.Lfunc_end0:
"""
    probs = A.audit_kernel(bad, "_Zk")
    assert len(probs) == 2 and "VALU write" in probs[0] and "MFMA" in probs[1]
    good = """_Zk:
\tv_mul_f32_e32 v4, v1, v2
\ts_nop 1
\tv_mfma_f32_16x16x32_f16 a[0:3], v[4:7], v[8:11], a[0:3]
\ts_nop 7
\ts_nop 7
\tv_accvgpr_read_b32 v20, a1
\ts_endpgm
.Lfunc_end0:
"""
    assert A.audit_kernel(good, "_Zk") == []


def test_expert_gemm_kernels_keep_the_mfma_waits(tmp_path):
    asm = A.asm_of_mlp(str(tmp_path))
    big = A.kernels(asm, r"k_expert_gemmILi8E")
    small = A.kernels(asm, r"k_expert_gemmILi4E")
    assert len(big) == 6 and len(small) == 6   # gate/up and down, three weight formats
    for k in big + small:
        assert A.audit_kernel(asm, k) == [], k
