"""The Python binding refuses device tensors the C ABI cannot check (wrong dtype,
non-contiguous, too small for the layout, misaligned) with TQ_ERR_INVALID before
the library is called, so nothing is launched on a bad buffer."""

import pytest
import torch

pytestmark = pytest.mark.gpu

tq = pytest.importorskip("compressed_domain_attention_kv_amd")


@pytest.fixture(scope="module")
def env():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = tq.Layout(2, 8, 2, 128, 256, tq.FMT_PQ4, tq.FMT_PQ4)
    cb, _ = tq.build_codebook(128, 4, 0, 1, 2)
    kb, vb = tq.cache_bytes(L)
    d = dict(L=L, cb=cb,
             kc=torch.zeros(kb, dtype=torch.uint8, device="cuda"), vc=torch.zeros(vb, dtype=torch.uint8, device="cuda"),
             q=torch.zeros(2, 8, 128, device="cuda"), out=torch.zeros(2, 8, 128, device="cuda"),
             sl=torch.full((2,), 100, dtype=torch.int32, device="cuda"), ws=tq.decode_workspace(L))
    yield d


def _refused(fn, match):
    with pytest.raises(tq.TQError, match=match) as e:
        fn()
    assert e.value.status == -1


def test_decode_attention_argument_checks(env):
    L, cb, kc, vc, q, out, sl, ws = (env[k] for k in ("L", "cb", "kc", "vc", "q", "out", "sl", "ws"))

    def call(**kw):
        a = dict(q_rot=q, k_cache=kc, v_cache=vc, seq_lens=sl, out=out, ws=ws)
        a.update(kw)
        return lambda: tq.decode_attention(L, cb, cb, a["q_rot"], None, a["k_cache"], a["v_cache"], a["seq_lens"],
                                           a["out"], a["ws"])

    _refused(call(seq_lens=sl.to(torch.int64)), "seq_lens must be torch.int32")
    _refused(call(q_rot=q.half()), "q_rot must be torch.float32")
    _refused(call(k_cache=kc[:-1]), "k_cache holds")
    _refused(call(v_cache=vc[4:]), "v_cache holds")
    _refused(call(out=torch.zeros(2, 8, 64, device="cuda")), "out holds")
    _refused(call(q_rot=torch.zeros(2, 128, 8, device="cuda").transpose(1, 2)), "q_rot must be contiguous")
    _refused(call(ws=ws[:-256]), "ws holds")
    mis = torch.zeros(kc.numel() + 16, dtype=torch.uint8, device="cuda")[4:4 + kc.numel()]
    _refused(call(k_cache=mis), "k_cache must be 16-byte aligned")
    _refused(call(seq_lens=sl.cpu()), "seq_lens must be a GPU tensor")
    call()()  # the well-formed call goes through
    torch.cuda.synchronize()


def test_write_and_step_argument_checks(env):
    L, cb, kc, vc, q, sl, ws = (env[k] for k in ("L", "cb", "kc", "vc", "q", "sl", "ws"))
    rows = torch.zeros(3, 2, 128, dtype=torch.float16, device="cuda")
    dst = torch.arange(3, dtype=torch.int32, device="cuda")
    _refused(lambda: tq.quantize_append(L, cb, cb, None, rows[:2], rows, dst, kc, vc), "k_new holds")
    _refused(lambda: tq.quantize_append(L, cb, cb, None, rows.float(), rows, dst, kc, vc),
             "k_new must be torch.float16")
    _refused(lambda: tq.quantize_append(L, cb, cb, None, rows, rows, dst.long(), kc, vc), "dst_row must be")
    new = torch.zeros(2, 2, 128, dtype=torch.float16, device="cuda")
    pos = torch.zeros(2, dtype=torch.int32, device="cuda")
    _refused(lambda: tq.decode_step(L, cb, cb, new, new, pos, q, torch.empty_like(q), kc, vc, sl, ws,
                                    out=torch.zeros(2, 8, 127, device="cuda")), "out holds")
    _refused(lambda: tq.decode_step(L, cb, cb, new[:1], new, pos, q, torch.empty_like(q), kc, vc, sl, ws),
             "k_new holds")
    ring = torch.zeros(tq.ring_bytes(L, 64) // 2, dtype=torch.float16, device="cuda")
    _refused(lambda: tq.ring_append(L, 64, new, new, pos, ring[:-1], ring), "k_ring holds")
