"""The two-level checkpoint loader: splitting the fused gate/up stack,
per-expert global scales, safetensors, rejects (CPU), and the device repack
of loaded stacks checked bit-exact against the oracle's decode (GPU)."""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import formats as F
from oracle.quantize import quantize_experts

E, I, H = 3, 32, 128


def _two_level(n, k, seed, per_expert=True):
    rng = np.random.default_rng(seed)
    w = S.f32_to_bf16_bits((rng.standard_normal((E, n, k)) * 0.02).astype(np.float32))
    packed, codes, g = quantize_experts(F.bf16_bits_to_f64(w))
    g2 = torch.from_numpy(np.asarray(g, np.float32).reshape(E, 1, 1)) if per_expert else \
        torch.tensor(float(g[0]), dtype=torch.float32)
    return torch.from_numpy(packed), torch.from_numpy(codes), g2


def _oracle_rows(p, s, g2, e, r0, r1):
    gv = g2.reshape(-1)
    gv = float(gv[e] if gv.numel() > 1 else gv[0])
    return F.dequantize(p[e, r0:r1].numpy(), s[e, r0:r1].numpy(), gv)


def test_split_rows_and_scales():
    from nvfp4_weight_only_moe_amd import checkpoint as C
    gu = _two_level(2 * I, H, 1)
    dn = _two_level(H, I, 2, per_expert=False)
    # weight_scale given as float8 bytes must load the same as u8
    gu8 = (gu[0], gu[1].view(torch.float8_e4m3fn), gu[2])
    for src in (gu, gu8):
        gate, up, down = C.load_experts(src, dn, device="cpu", tiled=False)
        for e in range(E):
            assert np.array_equal(F.dequantize(gate.packed[e].numpy(), gate.scales[e].numpy(),
                                               float(gate.global_scale[e])),
                                  _oracle_rows(*gu, e, 0, I))
            assert np.array_equal(F.dequantize(up.packed[e].numpy(), up.scales[e].numpy(),
                                               float(up.global_scale[e])),
                                  _oracle_rows(*gu, e, I, 2 * I))
            assert np.array_equal(F.dequantize(down.packed[e].numpy(), down.scales[e].numpy(),
                                               float(down.global_scale[e])),
                                  _oracle_rows(*dn, e, 0, H))
    assert (gate.N, gate.K, down.N, down.K) == (I, H, H, I)


def test_safetensors_round_trip(tmp_path):
    from safetensors.torch import save_file
    from nvfp4_weight_only_moe_amd import checkpoint as C
    gu, dn = _two_level(2 * I, H, 3), _two_level(H, I, 4)
    t = {"experts.gate_up_proj": gu[0], "experts.gate_up_proj.weight_scale": gu[1],
         "experts.gate_up_proj.weight_scale_2": gu[2].reshape(E).contiguous(),
         "experts.down_proj": dn[0], "experts.down_proj.weight_scale": dn[1],
         "experts.down_proj.weight_scale_2": dn[2].reshape(E).contiguous()}
    path = str(tmp_path / "experts.safetensors")
    save_file(t, path)
    a = C.load_experts_safetensors(path, "experts.gate_up_proj", "experts.down_proj",
                                   device="cpu", tiled=False)
    b = C.load_experts(gu, dn, device="cpu", tiled=False)
    for x, y in zip(a, b):
        assert torch.equal(x.packed, y.packed) and torch.equal(x.scales, y.scales)
        assert torch.equal(x.global_scale, y.global_scale)


def test_loader_rejects():
    from nvfp4_weight_only_moe_amd import checkpoint as C
    p, s, g = _two_level(2 * I, H, 5)
    with pytest.raises(ValueError):
        C.stack_from_two_level(p, s[:, :, :-1], g, device="cpu")          # scale shape
    with pytest.raises(ValueError):
        C.stack_from_two_level(p, s, torch.ones(E + 1), device="cpu")     # scale_2 count
    with pytest.raises(TypeError):
        C.stack_from_two_level(p.to(torch.int32), s, g, device="cpu")     # element size
    odd = C.stack_from_two_level(p[:, :-1], s[:, :-1], g, device="cpu")
    with pytest.raises(ValueError):
        C.split_gate_up(odd)                                               # odd fused rows
    dn = _two_level(H, I, 6)
    with pytest.raises(ValueError):
        C.load_experts((p, s, g), (dn[0][:, :64], dn[1][:, :64], dn[2]), device="cpu",
                       tiled=False)                                        # does not chain


@pytest.mark.gpu
def test_loaded_stacks_repack_bit_exact():
    import nvfp4_weight_only_moe_amd as moe
    from nvfp4_weight_only_moe_amd import checkpoint as C
    gu, dn = _two_level(2 * I, H, 7), _two_level(H, I, 8)
    gate, up, down = C.load_experts(gu, dn, device="cuda", tiled=True)
    torch.cuda.synchronize()
    for w, src, r0 in ((gate, gu, 0), (up, gu, I), (down, dn, 0)):
        assert w.layout == moe.LAYOUT_TILED
        for e in range(E):
            out = torch.empty((w.N, w.K), dtype=torch.bfloat16, device="cuda")
            moe.nvfp4_dequant_bf16(w, e, out)
            torch.cuda.synchronize()
            # the device check decodes E2M1 x E4M3 (exact in bf16); the global separately
            ref = F.dequantize_no_global(src[0][e, r0:r0 + w.N].numpy(),
                                         src[1][e, r0:r0 + w.N].numpy())
            got = out.float().cpu().numpy().astype(np.float64)
            assert np.array_equal(got, ref)
            g = src[2].reshape(-1)
            assert float(w.global_scale[e]) == float(g[e] if g.numel() > 1 else g[0])
