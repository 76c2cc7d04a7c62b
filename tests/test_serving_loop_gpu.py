"""A short serving loop on the GPU, driven by the library's native block manager, over 16-bit and
over E4M3 caches (lecture 34 "vLLM 生产级系统架构全景剖析" §4.4).

Requests share a system prompt (prefix cache), one request forks into parallel samples (copy on
write of its partly filled last block), requests finish and new ones reuse cached free blocks.
Every step runs the device path in order -- pa_copy_blocks for the manager's copy pairs,
pa_reshape_and_cache into the manager's slots, then pa_prefill_chunk / pa_decode over the
manager's block tables -- and is checked three ways:
  * the manager's slots, copy pairs and tables equal the plain-Python oracle manager's;
  * the GPU pools equal, word for word, the pools the CPU oracle's scatter and copy produce under
    the oracle manager's decisions;
  * the attention outputs equal the float64 oracle's attention over each sequence's CONTIGUOUS
    K/V rows, which are drawn from the token ids alone (row p from a generator seeded by a rolling
    hash of ids[0..p], as a model's K/V depend on the whole prefix). No block bookkeeping enters
    that reference, so a wrong slot, a stale reused block or a missed copy shows up there.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import OracleBlockManager
from pa_testutil import assert_attention_close
from pa_workloads import f32_to_words
from paged_kv_cache_99_amd import binding
from paged_kv_cache_99_amd.block_manager import BlockManager

pytestmark = pytest.mark.gpu

H_Q, H_KV, D, BLOCK = 8, 2, 128, 16
NAN_WORD = {"f16": 0x7E00, "bf16": 0x7FC0}
NAN_E4M3 = 0x7F
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16}
KS, VS = 0.03, 0.02  # E4M3 cache scales
_MOD = (1 << 61) - 1


class TokenRows:
    """K/V words of each position, a function of the token ids up to it."""

    def __init__(self, dtype):
        self.dtype = dtype
        self.memo = {}

    def rows(self, ids, start, stop):
        h, ks, vs = 0, [], []
        for p in range(stop):
            h = (h * 1000003 + int(ids[p]) + 1) % _MOD
            if p < start:
                continue
            if h not in self.memo:
                r = np.random.default_rng(h).standard_normal(2 * H_KV * D, dtype=np.float32)
                self.memo[h] = f32_to_words(r, self.dtype).reshape(2, H_KV, D)
            ks.append(self.memo[h][0])
            vs.append(self.memo[h][1])
        if not ks:
            e = np.zeros((0, H_KV, D), np.uint16)
            return e, e.copy()
        return np.stack(ks), np.stack(vs)


def reference_attention(q_words, ids, upto, rows: TokenRows, dtype, scale, fp8=False):
    """float64 [H_q][D]: the query of position upto-1 over contiguous rows 0..upto-1 (with fp8,
    the rows as E4M3 caches hold them: the codes of x / scale, times the scale)."""
    K, V = rows.rows(ids, 0, upto)
    if fp8:
        Kd = oracle.e4m3_to_double(oracle.quantize_e4m3(K, dtype, KS)) * KS
        Vd = oracle.e4m3_to_double(oracle.quantize_e4m3(V, dtype, VS)) * VS
    else:
        Kd, Vd = oracle.to_double(K, dtype), oracle.to_double(V, dtype)
    qd = oracle.to_double(q_words, dtype)
    g = H_Q // H_KV
    return np.stack([oracle.attention(qd[h], np.ascontiguousarray(Kd[:, h // g]),
                                      np.ascontiguousarray(Vd[:, h // g]), scale)
                     for h in range(H_Q)])


class Loop:
    def __init__(self, dtype, num_blocks, seed, fp8=False):
        self.dtype, self.nb, self.fp8 = dtype, num_blocks, fp8
        self.rng = np.random.default_rng(seed)
        order = self.rng.permutation(num_blocks)
        self.native = BlockManager(num_blocks, order, prefix_caching=True)
        self.ref = OracleBlockManager(num_blocks, order, prefix_caching=True)
        n = num_blocks * H_KV * BLOCK * D
        if fp8:
            self.kc_ref = np.full(n, NAN_E4M3, np.uint8)        # slots never written stay NaN
            self.kc = torch.from_numpy(self.kc_ref.copy()).cuda()
        else:
            self.kc_ref = np.full(n, NAN_WORD[dtype], np.uint16)
            self.kc = torch.from_numpy(self.kc_ref.view(np.int16).copy()).view(TORCH[dtype]).cuda()
        self.vc_ref = self.kc_ref.copy()
        self.kc = self.kc.view(num_blocks, H_KV, BLOCK, D)
        self.vc = self.kc.clone()
        self.rows = TokenRows(dtype)
        self.ids = {}
        self.scale = 1.0 / np.sqrt(D)

    def dev_words(self, a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            TORCH[self.dtype]).cuda()

    def i32(self, a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    def write(self, pairs, toks):
        """pairs: copy-on-write (src, dst); toks: (sid, first position, slots) of new tokens."""
        if pairs:
            m = np.array(pairs, np.int32)
            binding.copy_blocks(self.kc, self.vc, self.i32(m))
            copy = oracle.copy_blocks_fp8 if self.fp8 else oracle.copy_blocks
            self.kc_ref, self.vc_ref = copy(self.kc_ref, self.vc_ref, m, self.nb, H_KV, D)
        ks, vs, slots = [], [], []
        for sid, p0, sl in toks:
            k, v = self.rows.rows(self.ids[sid], p0, p0 + len(sl))
            ks.append(k)
            vs.append(v)
            slots.extend(sl)
        if not slots:
            return
        K, V, S = np.concatenate(ks), np.concatenate(vs), np.array(slots, np.int32)
        if self.fp8:
            binding.reshape_and_cache_fp8(self.dev_words(K), self.dev_words(V), self.kc, self.vc,
                                          self.i32(S), KS, VS)
            self.kc_ref, self.vc_ref = oracle.reshape_and_cache_fp8(
                K, V, self.kc_ref, self.vc_ref, S, self.nb, H_KV, D, self.dtype, KS, VS)
        else:
            binding.reshape_and_cache(self.dev_words(K), self.dev_words(V), self.kc, self.vc,
                                      self.i32(S))
            self.kc_ref, self.vc_ref = oracle.reshape_and_cache(K, V, self.kc_ref, self.vc_ref, S,
                                                                self.nb, H_KV, D)

    def both(self, fn, *args):
        a = getattr(self.native, fn)(*args)
        b = getattr(self.ref, fn)(*args)
        if fn == "allocate_slots":
            a = (list(map(int, a[0])), a[1])
        assert a == b, (fn, args, a, b)
        return b

    def tables(self, sids):
        mb = max(self.ref.sequence_info(s)[1] for s in sids)
        t = self.native.block_tables(sids, mb)
        assert t.tolist() == [self.ref.block_table(s) + [-1] * (mb - len(self.ref.block_table(s)))
                              for s in sids]
        return t

    def admit(self, prompts):
        """New requests: prefix match, slots for the rest, scatter, one prefill call."""
        toks, pairs, rows = [], [], []
        for sid, prompt in prompts:
            self.ids[sid] = list(prompt)
            self.both("add_sequence", sid)
            hit = self.both("match_prefix", sid, prompt)
            slots, pair = self.both("allocate_slots", sid, len(prompt) - hit, prompt[hit:])
            assert pair is None
            toks.append((sid, hit, slots))
            rows.append((sid, hit, len(prompt)))
        self.write(pairs, toks)
        sids = [s for s, _, _ in rows]
        q_lens = [n - h for _, h, n in rows]
        cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        q = f32_to_words(self.rng.standard_normal((int(cu[-1]), H_Q, D), dtype=np.float32),
                         self.dtype)
        out = torch.empty((int(cu[-1]), H_Q, D), dtype=TORCH[self.dtype], device="cuda")
        args = (out, self.dev_words(q), self.kc, self.vc, self.i32(self.tables(sids)),
                self.i32([n for _, _, n in rows]), self.i32(cu), max(q_lens), self.scale)
        if self.fp8:
            binding.prefill_chunk_fp8(*args, KS, VS)
        else:
            binding.prefill_chunk(*args)
        got = out.cpu().view(torch.int16).numpy().view(np.uint16)
        ref = np.stack([reference_attention(q[cu[i] + j], self.ids[sid], h + j + 1, self.rows,
                                            self.dtype, self.scale, self.fp8)
                        for i, (sid, h, n) in enumerate(rows) for j in range(n - h)])
        self.check_pools()
        assert_attention_close(got, ref, self.dtype, f"prefill {sids}")
        return [h for _, h, _ in rows]

    def decode_step(self, sids, partition_size):
        toks, pairs = [], []
        for sid in sids:
            tok = int(self.rng.integers(0, 50))
            p0 = len(self.ids[sid])
            self.ids[sid].append(tok)
            slots, pair = self.both("allocate_slots", sid, 1, [tok])
            if pair is not None:
                pairs.append(pair)
            toks.append((sid, p0, slots))
        self.write(pairs, toks)
        lens = [len(self.ids[s]) for s in sids]
        q = f32_to_words(self.rng.standard_normal((len(sids), H_Q, D), dtype=np.float32),
                         self.dtype)
        out = torch.empty((len(sids), H_Q, D), dtype=TORCH[self.dtype], device="cuda")
        if self.fp8:
            binding.decode_fp8(out, self.dev_words(q), self.kc, self.vc, self.i32(self.tables(sids)),
                               self.i32(lens), max(lens), self.scale, KS, VS,
                               partition_size=partition_size)
        else:
            binding.decode(out, self.dev_words(q), self.kc, self.vc, self.i32(self.tables(sids)),
                           self.i32(lens), max(lens), self.scale, partition_size=partition_size)
        got = out.cpu().view(torch.int16).numpy().view(np.uint16)
        ref = np.stack([reference_attention(q[i], self.ids[s], lens[i], self.rows, self.dtype,
                                            self.scale, self.fp8) for i, s in enumerate(sids)])
        self.check_pools()
        assert_attention_close(got, ref, self.dtype, f"decode {sids}")
        return len(pairs)

    def check_pools(self):
        torch.cuda.synchronize()
        for dev, ref in ((self.kc, self.kc_ref), (self.vc, self.vc_ref)):
            if self.fp8:
                words = dev.cpu().numpy().ravel()
            else:
                words = dev.cpu().view(torch.int16).numpy().view(np.uint16).ravel()
            assert np.array_equal(words, ref), "pool differs from the oracle's"

    def fork(self, parent, child):
        self.both("fork", parent, child)
        self.ids[child] = list(self.ids[parent])

    def free(self, sid):
        self.both("free", sid)
        del self.ids[sid]


@pytest.mark.parametrize("dtype,partition_size,kv", [("f16", 0, "auto"), ("bf16", 32, "auto"),
                                                     ("f16", 32, "fp8"), ("bf16", 0, "fp8")])
def test_serving_loop_with_native_block_manager(dtype, partition_size, kv):
    print(f"[serving loop] dtype={dtype} partition={partition_size} kv={kv}", flush=True)
    L = Loop(dtype, num_blocks=64, seed=5, fp8=kv == "fp8")
    system = [int(x) for x in L.rng.integers(0, 50, 40)]      # 2.5 blocks of shared prompt
    qs = [[int(x) for x in L.rng.integers(0, 50, n)] for n in (9, 23, 4, 17)]
    hits = L.admit([(0, system + qs[0]), (1, system + qs[1])])
    # request 0's full blocks enter the cache as it is admitted, so request 1, admitted after it in
    # the same call, already shares the two whole blocks of the system prompt (written by the same
    # scatter before the prefill reads them)
    assert hits == [0, 32]
    hits = L.admit([(2, system + qs[2])])
    assert hits == [32]                      # the two whole blocks of the system prompt
    L.fork(2, 3)                             # parallel samples of request 2 (44 tokens: partial)
    L.fork(2, 4)
    copies = 0
    live = [0, 1, 2, 3, 4]
    for step in range(14):
        copies += L.decode_step(live, partition_size)
        if step == 4:
            L.free(1)                        # request 1 finishes; its blocks become cached free
            live.remove(1)
            hits = L.admit([(5, system + qs[1])])
            assert hits == [48]              # system prompt + question 1 up to its last block
            live.append(5)
        if step == 9:
            L.free(0)
            live.remove(0)
            hits = L.admit([(6, system + qs[3])])
            assert hits == [32]
            live.append(6)
    assert copies == 2                       # two of the three samples copied the shared block
    for sid in live:
        L.free(sid)
    assert L.native.num_free_blocks == 64
