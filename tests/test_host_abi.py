"""Host-side checks of libdsa that need no GPU: the shared library loads and exports every
function include/dsa.h declares; the config rules, geometry helpers, host weight transforms
and bf16 rounding agree with the oracle; and every argument refusal returns its code
without launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from dsa_pooled_key_amd import binding as dsa
from dsa_pooled_key_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return [l.split() for l in fh if l.strip() and not l.startswith("#")]


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = dsa.lib()
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dsa.EXPORTED)
    assert dsa.version().startswith("dsa ")


def _cfg(**kw):
    base = dict(index_heads=32, index_head_dim=128, index_kpool=4, index_topk=2048, heads=32)
    base.update(kw)
    return dsa.Config.make(**base)


RULE_TO_CODE = {0: 0, 1: -4, 2: -5, 3: -6, 4: -7, 5: -8, 6: -9}


def test_validate_matches_oracle_and_page_order():
    for kp, tk, kvl, heads, rule in _rows("validate_cases.txt"):
        cfg = _cfg(index_kpool=int(kp), index_topk=int(tk), kv_lora_rank=int(kvl),
                   heads=int(heads))
        assert dsa.config_validate(cfg) == RULE_TO_CODE[int(rule)], (kp, tk, kvl, heads)
        assert oracle.validate(int(kp), int(tk), int(kvl), int(heads)) == int(rule)


def test_geometry_matches_oracle():
    for tk, kp, n, tail, sk, ow in _rows("geometry_cases.txt"):
        cfg = _cfg(index_kpool=int(kp), index_topk=int(tk), always_select_tail=bool(int(tail)))
        assert dsa.select_k(cfg, int(n)) == int(sk) == oracle.select_k(int(tk), int(kp), int(n))
        assert dsa.out_width(cfg) == int(ow)
    for S, f, kp in [(1024, 0, 4), (1023, 0, 4), (1024, 3, 4), (3, 0, 4), (262144, 0, 4),
                     (131072, 0, 8), (5, 5, 1)]:
        assert dsa.num_pools(S, f, kp) == oracle.num_pools(S, f, kp)
    with pytest.raises(dsa.DsaError):
        dsa.num_pools(10, 0, 0)


def _absorb_case(seed, heads=3, nope=8, vd=6, kvl=512, ql=24, hidden=10):
    rng = np.random.default_rng(seed)
    q_b = rng.standard_normal((heads * nope, ql)).astype(np.float32)
    kv_b = rng.standard_normal((heads * (nope + vd), kvl)).astype(np.float32)
    o = rng.standard_normal((hidden, heads * vd)).astype(np.float32)
    cfg = _cfg(qk_nope_head_dim=nope, v_head_dim=vd, q_lora_rank=ql, hidden=hidden, heads=heads)
    return cfg, q_b, kv_b, o


def test_absorb_q_is_thread_count_invariant_and_equals_oracle(monkeypatch):
    cfg, q_b, kv_b, _ = _absorb_case(1)
    H = 3
    ref = oracle.absorb_q(q_b, kv_b, heads=H, nope=8, rope=0, vd=6, kvl=512, ql=24)
    rows = H * 512
    for t in (1, 2, 3, 7, 64, rows, rows + 5):
        got = dsa.absorb_q(cfg, q_b, kv_b, full_heads=H, threads=t)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), t
    for env in ("5", " 3 ", "0", "-2", "abc", ""):
        monkeypatch.setenv("DSA_ABSORB_THREADS", env)
        got = dsa.absorb_q(cfg, q_b, kv_b, full_heads=H, threads=0)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), env


def test_absorb_o_is_thread_count_invariant_and_equals_oracle():
    cfg, _, kv_b, o = _absorb_case(2)
    ref = oracle.absorb_o(o, kv_b, heads=3, nope=8, rope=0, vd=6, kvl=512, hidden=10)
    for t in (1, 2, 4, 10, 0):
        got = dsa.absorb_o(cfg, o, kv_b, local_heads=3, threads=t)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), t


@pytest.mark.parametrize("threads", [1, 3, 0])
def test_absorb_several_column_blocks_equal_oracle(threads):
    """Widths that cut the product's tiles raggedly (q_lora_rank 200 and hidden 150 over
    64-column blocks, two heads): bit-identical to the oracle's per-element sums at one,
    three and all threads."""
    cfg, q_b, kv_b, o = _absorb_case(7, heads=2, nope=16, vd=12, kvl=512, ql=200, hidden=150)
    rq = oracle.absorb_q(q_b, kv_b, heads=2, nope=16, rope=0, vd=12, kvl=512, ql=200)
    ro = oracle.absorb_o(o, kv_b, heads=2, nope=16, rope=0, vd=12, kvl=512, hidden=150)
    gq = dsa.absorb_q(cfg, q_b, kv_b, full_heads=2, threads=threads)
    go = dsa.absorb_o(cfg, o, kv_b, local_heads=2, threads=threads)
    assert np.array_equal(gq.view(np.uint32), rq.view(np.uint32))
    assert np.array_equal(go.view(np.uint32), ro.view(np.uint32))


def test_absorb_refusals():
    cfg, q_b, kv_b, o = _absorb_case(3)
    with pytest.raises(dsa.DsaError) as e:
        dsa.absorb_q(cfg, q_b[:-1], kv_b, full_heads=3)
    assert e.value.code == -11
    with pytest.raises(dsa.DsaError) as e:
        dsa.absorb_q(cfg, q_b, kv_b[:-1], full_heads=3)
    assert e.value.code == -11
    rope = _cfg(qk_nope_head_dim=8, v_head_dim=6, q_lora_rank=24, hidden=10, heads=3,
                qk_rope_head_dim=2)
    qr = np.zeros((3 * 10, 24), np.float32)
    with pytest.raises(dsa.DsaError) as e:
        dsa.absorb_q(rope, qr, kv_b, full_heads=3)
    assert e.value.code == -10
    with pytest.raises(dsa.DsaError) as e:
        dsa.absorb_o(rope, o, kv_b, local_heads=3)
    assert e.value.code == -10
    with pytest.raises(dsa.DsaError) as e:
        dsa.absorb_o(cfg, o[:, :-1], kv_b, local_heads=3)
    assert e.value.code == -11


def test_bf16_rounding_matches_oracle_and_generator():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(4096) * np.exp2(rng.integers(-30, 30, 4096))).astype(np.float32)
    x[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 65504.0]
    got = dsa.f32_to_bf16_rne(x)
    assert np.array_equal(got, synth.bf16_bits(x))
    assert all(int(got[i]) == oracle.bf16_from_float(float(x[i])) for i in range(0, 4096, 37))
    assert got[0] == 0x3F80 and got[1] == 0x3F82


# ---------------------------------------------------------------- refusals, no launch

_NULL = None
_FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below is refused first


def test_measurement_entry_points_refuse_bad_arguments():
    """The measurement-only calls check their arguments before any launch."""
    L = dsa.lib()
    assert L.dsa_empty_launch(0, _NULL) == -2
    assert L.dsa_empty_launch(65536, _NULL) == -2
    assert L.dsa_mfma_rate(3, 1, 2, _FAKE, _NULL) == -2      # no such shape
    assert L.dsa_mfma_rate(0, 0, 2, _FAKE, _NULL) == -2      # no blocks
    assert L.dsa_mfma_rate(1, 1, 3, _FAKE, _NULL) == -2      # odd round count
    assert "even" in dsa.last_error()
    assert L.dsa_mfma_rate(2, 1, 2, _NULL, _NULL) == -1      # no output
    assert L.dsa_stream_read(_FAKE, 24, _FAKE, _NULL) == -2  # not a multiple of 16 bytes
    assert L.dsa_stream_read(_NULL, 32, _FAKE, _NULL) == -1
    assert L.dsa_stream_read(_NULL, 0, _NULL, _NULL) == 0     # nothing to read


def test_refusals_return_codes_without_launching():
    L = dsa.lib()
    cfg = _cfg()
    c = ctypes.byref(cfg)
    bad = _cfg(index_kpool=9, index_topk=9)
    # config rules reach every call
    assert L.dsa_index_scores(ctypes.byref(bad), 1, 1, 8, 0, 1.0, _FAKE, _FAKE, _FAKE, _FAKE,
                              _FAKE, 0, _NULL, _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -6
    # null buffers
    assert L.dsa_index_scores(c, 1, 1, 8, 0, 1.0, _NULL, _FAKE, _FAKE, _FAKE, _FAKE, 0, _NULL,
                              _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -1
    assert "NULL" in dsa.last_error()
    # fp8 keys without scales; bad dtype
    assert L.dsa_index_scores(c, 1, 1, 8, 0, 1.0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 2, _NULL,
                              _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -1
    assert L.dsa_index_scores(c, 1, 1, 8, 0, 1.0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, 1, _NULL,
                              _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -3
    # unsupported indexer geometry
    assert L.dsa_index_scores(ctypes.byref(_cfg(index_head_dim=48)), 1, 1, 8, 0, 1.0, _FAKE,
                              _FAKE, _FAKE, _FAKE, _FAKE, 0, _NULL, _FAKE, _FAKE, _FAKE, _FAKE,
                              _NULL) == -14
    assert L.dsa_index_scores(ctypes.byref(_cfg(index_heads=33)), 1, 1, 8, 0, 1.0, _FAKE,
                              _FAKE, _FAKE, _FAKE, _FAKE, 0, _NULL, _FAKE, _FAKE, _FAKE, _FAKE,
                              _NULL) == -14
    # misaligned data pointer
    odd = ctypes.c_void_p(0x10002)
    assert L.dsa_index_scores(c, 1, 1, 8, 0, 1.0, odd, _FAKE, _FAKE, _FAKE, _FAKE, 0, _NULL,
                              _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -2
    # top-k rows beyond the register budget
    assert L.dsa_topk_pools(c, 1, 65537, _FAKE, _FAKE, _FAKE, _NULL, 0, _NULL) == -14
    # a workspace size without a pointer
    assert L.dsa_topk_pools(c, 1, 16384, _FAKE, _FAKE, _FAKE, _NULL, 4096, _NULL) == -12
    # expand: more pools than the index_topk budget
    assert L.dsa_expand_selection(c, 1, 513, 1, 4096, 0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE,
                                  _NULL) == -2
    # kpool_compress negative size / null
    assert L.dsa_kpool_compress(c, 1, -1, 0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE,
                                _NULL) == -2
    assert L.dsa_kpool_compress(c, 1, 64, 0, _NULL, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE,
                                _NULL) == -1
    # sparse MLA: missing workspace when the plan splits
    need = L.dsa_sparse_mla_decode_workspace(c, 32, 4096)
    assert need > 0
    assert L.dsa_sparse_mla_decode(c, 32, 4096, 32, 0.0625, _FAKE, _FAKE, _FAKE, _FAKE, 0,
                                   _NULL, 1 << 20, 131072, _NULL, 0, 64, _FAKE, _NULL, _NULL, 0,
                                   _NULL) == -12
    assert L.dsa_sparse_mla_decode(c, 32, 4096, 32, 0.0625, _FAKE, _FAKE, _FAKE, _FAKE, 2,
                                   _NULL, 1 << 20, 131072, _NULL, 0, 64, _FAKE, _NULL, _FAKE,
                                   need, _NULL) == -1
    # a contiguous latent (no block table) needs a positive stride S: with S = 0 every
    # sequence would read sequence 0's rows
    for S in (0, -1):
        assert L.dsa_sparse_mla_decode(c, 2, 8, 2, 0.0625, _FAKE, _FAKE, _FAKE, _FAKE, 0, _NULL,
                                       1 << 20, S, _NULL, 0, 64, _FAKE, _NULL, _NULL, 0,
                                       _NULL) == -2
    # paged, S = 0 only means no bound on the token ids: accepted up to the workspace check
    assert L.dsa_sparse_mla_decode(c, 32, 4096, 32, 0.0625, _FAKE, _FAKE, _FAKE, _FAKE, 0,
                                   _NULL, 1 << 20, 0, _FAKE, 2048, 64, _FAKE, _NULL, _NULL, 0,
                                   _NULL) == -12
    assert L.dsa_sparse_mla_decode(ctypes.byref(_cfg(kv_lora_rank=576)), 1, 8, 1, 0.0625, _FAKE,
                                   _FAKE, _FAKE, _FAKE, 0, _NULL, 64, 64, _NULL, 0, 64, _FAKE,
                                   _NULL, _NULL, 0, _NULL) == -8
    # empty work is accepted and launches nothing
    assert L.dsa_index_scores(c, 0, 1, 8, 0, 1.0, _NULL, _NULL, _NULL, _NULL, _NULL, 0, _NULL,
                              _NULL, _NULL, _NULL, _NULL, _NULL) == 0
    assert L.dsa_compact_pools(0, 8, _NULL, _NULL, _NULL, _NULL) == 0


def test_sparse_mla_workspace_never_needs_more_than_sixteen_partials():
    """The split merge is built for 2 to 16 partials per (row, head group): the workspace the
    library asks for (one 33,024-byte partial per part) stays within that for every width up
    to the widest selection the boundary takes, from one row to prefill-sized batches."""
    L = dsa.lib()
    part = 256 + 32 * 512 * 2
    for heads in (32, 40):
        c = ctypes.byref(_cfg(heads=heads))
        groups = (heads + 31) // 32
        for Q in (1, 2, 8, 32, 64, 128, 256, 2048):
            for W in (1, 63, 64, 65, 1000, 2048, 4096, 4103, 16384, 32767, 32768):
                ws = L.dsa_sparse_mla_decode_workspace(c, Q, W)
                assert ws % (Q * groups * part) == 0
                parts = ws // (Q * groups * part)
                assert parts == 0 or 2 <= parts <= 16, (heads, Q, W, parts)


def test_refusals_of_the_fp8_writers_upkeep_and_masked_check():
    """Refused before any launch (no GPU needed): shapes the kernels are not built for, null
    buffers, bad dtypes, negative sizes."""
    L = dsa.lib()
    cfg = _cfg()
    c = ctypes.byref(cfg)
    # fp8 pooling: D not a power of two; null scales
    assert L.dsa_kpool_compress_fp8(ctypes.byref(_cfg(index_head_dim=48)), 1, 64, 0, _FAKE, _FAKE,
                                    _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -14
    assert L.dsa_kpool_compress_fp8(c, 1, 64, 0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, _FAKE,
                                    _NULL) == -1
    # quantizer: n not a multiple of 8, too wide, bad dtype, negative rows
    assert L.dsa_quantize_rows_fp8(4, 12, _FAKE, 0, _FAKE, _FAKE, _NULL) == -14
    assert L.dsa_quantize_rows_fp8(4, 4104, _FAKE, 0, _FAKE, _FAKE, _NULL) == -14
    assert L.dsa_quantize_rows_fp8(4, 512, _FAKE, 2, _FAKE, _FAKE, _NULL) == -3
    assert L.dsa_quantize_rows_fp8(-1, 512, _FAKE, 0, _FAKE, _FAKE, _NULL) == -2
    assert L.dsa_quantize_rows_fp8(0, 512, _NULL, 0, _NULL, _NULL, _NULL) == 0
    # k_norm: D not 8 times a power of two; negative eps
    assert L.dsa_k_norm(4, 96, _FAKE, _FAKE, _FAKE, ctypes.c_float(1e-5), _NULL) == -14
    assert L.dsa_k_norm(4, 128, _FAKE, _FAKE, _FAKE, ctypes.c_float(-1.0), _NULL) == -2
    # indexer_store / write_geom / pool_append nulls
    assert L.dsa_indexer_store(2, 8, 128, _NULL, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL) == -1
    assert L.dsa_write_geom(2, _FAKE, _NULL, _FAKE, _NULL) == -1
    assert L.dsa_pool_append(c, 2, 64, 0, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _FAKE, _NULL, _FAKE,
                             _NULL, _FAKE, _NULL) == -1
    # masked attention: more keys than the score row holds; fp8 without scales
    assert L.dsa_mla_masked_attn(c, 1, 32769, 1, ctypes.c_float(0.0625), _FAKE, _FAKE, _FAKE,
                                 _FAKE, 0, _NULL, 1 << 20, _NULL, 0, 64, _FAKE, _NULL,
                                 _NULL) == -14
    assert L.dsa_mla_masked_attn(c, 1, 64, 1, ctypes.c_float(0.0625), _FAKE, _FAKE, _FAKE, _FAKE,
                                 2, _NULL, 64, _NULL, 0, 64, _FAKE, _NULL, _NULL) == -1
    assert L.dsa_topk_to_mask(1, 4, 64, _FAKE, _NULL, _NULL) == -1


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asked for more it prints why and exits with status 2, before
    it touches a device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300, cwd=root)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
