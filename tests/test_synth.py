"""The seeded input generator on the CPU: stream slices regenerate identically, and the
sharing workloads realise the distinct-expert counts the pages give for six tokens."""
import numpy as np

import oracle.moe as omoe
import synth


def test_streams_regenerate_by_slice():
    cfg = synth.deepseek_v4_flash(8)
    a_codes, a_scales = synth.mxfp4_weights(cfg, "w2", 3, 3)
    b_codes, b_scales = synth.mxfp4_weights(cfg, "w2", 4, 1)
    assert np.array_equal(a_codes[1], b_codes[0]) and np.array_equal(a_scales[1], b_scales[0])
    assert a_scales.min() >= synth.MX_SCALE_LO and a_scales.max() < synth.MX_SCALE_LO + synth.MX_SCALE_SPAN
    x = synth.activations(synth.tiny())
    assert np.array_equal(x[5:9], synth.normal_bf16(101, synth.STREAM_X, 5 * 256, 4 * 256).reshape(4, 256))


def test_sharing_workloads_match_the_pages():
    """b12x README, "DeepSeek V4 Flash 0731 MoE reproduction": at six tokens the sharing
    levels 0, 20, 40, 60 and 80% have 36, 29, 22, 14 and 7 distinct experts, and 100%
    reaches the six-expert floor; no expert repeats inside a token. The router (with its
    selection bias) picks exactly the designated experts."""
    want = {0.0: 36, 0.2: 29, 0.4: 22, 0.6: 14, 0.8: 7, 1.0: 6}
    for level, n in want.items():
        cfg = synth.deepseek_v4_flash_sharing(6, level)
        picks = synth.sharing_experts(cfg)
        assert len(np.unique(picks)) == n
        assert all(len(set(r)) == cfg.k for r in picks.tolist())
        ids, _ = omoe.route(cfg, synth.logits(cfg))
        assert np.array_equal(np.sort(ids, 1), np.sort(picks, 1))
