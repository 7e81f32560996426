"""llm_sample_logits_static, the sampler entry point that allocates nothing
(its probability rows live in a static device buffer), against the handle's
llm_sample_d on the same logits and uniforms: identical token ids, on two
calls in a row, the second with a smaller input.  Both calls take the
two-launch path (vocabulary above 32768), which is the one that uses the
buffer.  The draws are also checked against the oracle's sampler."""
import numpy as np
import pytest

import oracle
from llama_decoder_forward_amd import synth
from tests.gpu_util import say
from tests.test_gpu_sampler import near_edge

pytestmark = [pytest.mark.gpu]


def test_static_sampler_matches_handle_sampler():
    import torch
    from llama_decoder_forward_amd import binding as B
    f = B.llm_sample_logits_static
    for V, nb, t, p in [(40000, 4, 0.6, 0.9), (36000, 2, 0.8, 0.95)]:
        say("static sampler: vocab", V, "rows", nb)
        kw = dict(n_layers=1, dim=256, n_heads=2, n_kv_heads=2, vocab_size=V, multiple_of=64,
                  max_batch_size=nb, max_seq_len=64, dtype=B.LLM_F16)
        h = B.llm_create(B.make_params(**kw), 71 + nb)
        h.prefill(synth.tokens(71 + nb, nb, 8, V))
        logits = torch.empty((nb, V), dtype=torch.float32, device="cuda")
        h.get_logits_d(logits.data_ptr())
        h.sync()
        lg = logits.cpu().numpy()
        for k in range(3):
            u_host = synth.uniforms(81 + V, 3, nb)[k]
            u = torch.from_numpy(u_host).cuda()
            out_h = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
            out_s = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
            torch.cuda.synchronize()
            h.sample_d(t, p, u.data_ptr(), out_h.data_ptr())
            h.sync()
            f(logits.data_ptr(), nb, V, t, p, u.data_ptr(), out_s.data_ptr(), h.stream())
            h.sync()
            a, b = out_h.cpu().numpy(), out_s.cpu().numpy()
            assert np.array_equal(a, b), (a, b)
            want = np.array([oracle.sample(lg[r], t, p, float(u_host[r])) for r in range(nb)])
            for r in np.nonzero(b != want)[0]:
                assert near_edge(lg[r], t, p, float(u_host[r]))
        # greedy needs no buffer
        out_s = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        f(logits.data_ptr(), nb, V, 0.0, 1.0, 0, out_s.data_ptr(), h.stream())
        h.sync()
        assert np.array_equal(out_s.cpu().numpy(), lg.argmax(-1))
        h.destroy()
    # a size beyond the buffer is refused before any launch
    with pytest.raises(B.LlmError) as ei:
        f(logits.data_ptr(), 200, 40000, 0.6, 0.9, u.data_ptr(), out_s.data_ptr())
    assert ei.value.code == B.LLM_EINVAL and "exceeds the static probability buffer" in str(ei.value)
