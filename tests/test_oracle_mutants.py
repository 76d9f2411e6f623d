"""Plant plausible mistakes in the oracle (on the CPU) and check that its pins catch
each one. Each mutant replaces one oracle function for the duration of a test."""
import math
from collections import deque

import numpy as np
import pytest

import oracle.attention as att
import oracle.block_manager as obm
import oracle.footprint as fp
import oracle.layout as layout
from tests import test_oracle_attention as TA
from tests import test_oracle_block_manager as TB
from tests import test_oracle_footprint as TF
from tests import test_oracle_kv_ops as TK


def _attend_mod_groups(q, K, V, scale):
    Hq, d = q.shape
    S, Hkv, _ = K.shape
    out = np.zeros((Hq, d))
    for h in range(Hq):
        g = h % Hkv                                   # wrong: strided instead of contiguous groups
        s = scale * (K[:, g, :] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


def _attend_no_scale(q, K, V, scale):
    return att_orig_attend(q, K, V, 1.0)


def _v_tile_untransposed(v_pool, layer, phys, head):
    return v_pool[layer, phys, head, :, :]


def _rebuild_short(k_pool, v_pool, layer, table, length, block_size, dtype):
    K, V = rebuild_orig(k_pool, v_pool, layer, table, length, block_size, dtype)
    if length > 1:
        K[-1] = K[-2]                                 # wrong: last token replaced by its neighbour
    return K, V


def _merge_wrong_sign(m_prev, l_prev, O_prev, m_blk, l_blk, O_blk):
    m_new = max(m_prev, m_blk)
    a = math.exp(m_new - m_prev) if m_prev != -math.inf else 0.0   # wrong sign
    b = math.exp(m_blk - m_new)
    return m_new, l_prev * a + l_blk * b, O_prev * a + O_blk * b


def _bytes_per_token_no_kv_factor(L, H, d, b, tp=1):
    return L * max(1, -(-H // tp)) * d * b


att_orig_attend = att.attend
rebuild_orig = att.rebuild_sequence


class _LifoDeque(deque):
    def popleft(self):
        return self.pop()


def _append_without_cow(self, sid, n):
    saved = self.ref[:]
    try:
        self.ref = [min(r, 1) for r in self.ref]     # wrong: never sees a shared tail
        return orig_append(self, sid, n)
    finally:
        for i, r in enumerate(saved):
            if r > 1:
                self.ref[i] = r


orig_append = obm.BlockManager.append


def _raises(fn, *args):
    """The pin must fail: by a failed assertion, or by the mutant's shapes not fitting."""
    with pytest.raises((AssertionError, ValueError)):
        fn(*args)


def test_mutant_gqa_mapping(monkeypatch):
    monkeypatch.setattr(att, "attend", _attend_mod_groups)
    _raises(TA.test_gqa_groups_are_contiguous)


def test_mutant_missing_scale(monkeypatch):
    monkeypatch.setattr(att, "attend", _attend_no_scale)
    _raises(TA.test_two_keys_weights_one_to_three_pin_the_scale)
    _raises(TA.test_brute_force_tiny, 16)


def test_mutant_v_layout(monkeypatch):
    monkeypatch.setattr(layout, "read_v_tile", _v_tile_untransposed)
    _raises(TK.test_tiny_rebuild)
    _raises(TA.test_brute_force_tiny, 4)


def test_mutant_dropped_token(monkeypatch):
    monkeypatch.setattr(att, "rebuild_sequence", _rebuild_short)
    _raises(TA.test_brute_force_tiny, 16)
    _raises(TK.test_appended_history_reads_back_exactly)


def test_mutant_online_merge_sign(monkeypatch):
    monkeypatch.setattr(att, "_merge", _merge_wrong_sign)
    _raises(TA.test_online_split_equals_direct, 100)


def test_mutant_footprint_factor(monkeypatch):
    monkeypatch.setattr(fp, "bytes_per_token", _bytes_per_token_no_kv_factor)
    _raises(TF.test_bytes_per_token, TF.GOLD["bytes_per_token"][0])


def test_mutant_lifo_free_list(monkeypatch):
    orig_init = obm.BlockManager.__init__

    def init(self, *a, **k):
        orig_init(self, *a, **k)
        self.free = _LifoDeque(self.free)
    monkeypatch.setattr(obm.BlockManager, "__init__", init)
    _raises(TB.test_figure5, "figure5_boundary")


def test_mutant_no_copy_on_write(monkeypatch):
    monkeypatch.setattr(obm.BlockManager, "append", _append_without_cow)
    _raises(TB.test_p3_fork_example)
    _raises(TB.test_figure5, "figure5_cow")


# ---------------------------------------------------------------------------
# Chunked prefill oracle
import oracle.prefill as opf  # noqa: E402
from tests import test_oracle_prefill as TP  # noqa: E402


def _chunk_attention_off_by_one(q_rows, k_rows, v_rows, K_hist, V_hist, scale):
    K_all = np.concatenate([K_hist, k_rows], axis=0)
    V_all = np.concatenate([V_hist, v_rows], axis=0)
    c = K_hist.shape[0]
    out = np.zeros(q_rows.shape)
    for t in range(q_rows.shape[0]):
        visible = c + t                               # wrong: a token does not see itself
        out[t] = att.attend(q_rows[t], K_all[:visible], V_all[:visible], scale)
    return out


def _chunk_attention_no_causal(q_rows, k_rows, v_rows, K_hist, V_hist, scale):
    K_all = np.concatenate([K_hist, k_rows], axis=0)
    V_all = np.concatenate([V_hist, v_rows], axis=0)
    return np.stack([att.attend(q_rows[t], K_all, V_all, scale)   # wrong: sees later chunk tokens
                     for t in range(q_rows.shape[0])])


def _chunk_attention_no_history(q_rows, k_rows, v_rows, K_hist, V_hist, scale):
    return chunk_attention_orig(q_rows, k_rows, v_rows, K_hist[:0], V_hist[:0], scale)


def _chunk_slots_relative(tables, q_start, ctx_lens, block_size):
    return chunk_slots_orig(tables, q_start, [0] * len(ctx_lens), block_size)  # wrong: ignores history


chunk_attention_orig = opf.chunk_attention
chunk_slots_orig = opf.chunk_slots


def test_mutant_prefill_causal_off_by_one(monkeypatch):
    monkeypatch.setattr(opf, "chunk_attention", _chunk_attention_off_by_one)
    _raises(TP.test_empty_history_is_causal_self_attention, 16)
    _raises(TP.test_one_token_chunks_equal_decode)


def test_mutant_prefill_no_causal_mask(monkeypatch):
    monkeypatch.setattr(opf, "chunk_attention", _chunk_attention_no_causal)
    _raises(TP.test_empty_history_is_causal_self_attention, 4)
    _raises(TP.test_chunked_equals_monolithic, 5)


def test_mutant_prefill_history_dropped(monkeypatch):
    monkeypatch.setattr(opf, "chunk_attention", _chunk_attention_no_history)
    _raises(TP.test_history_visible_and_chunk_causal)
    _raises(TP.test_brute_force_tiny)


def test_mutant_prefill_slots_relative(monkeypatch):
    monkeypatch.setattr(opf, "chunk_slots", _chunk_slots_relative)
    _raises(TP.test_chunk_written_at_table_positions)
    _raises(TP.test_chunked_equals_monolithic, 16)


# ---------------------------------------------------------------------------
# Tiered residency (asynchronous swapping)
from tests import test_oracle_tiering as TT  # noqa: E402


def _finish_to_front(self, sid, logical):
    self._check_logical(sid, logical)
    pend = self.pending.get(sid, {})
    for lb in logical:
        if pend.get(lb, ("",))[0] != "out":
            raise obm.InvalidArgument("nothing in flight")
    host = self.host.setdefault(sid, {})
    for lb in logical:
        _, p, frame = pend.pop(lb)
        self.ref[p] -= 1
        if self.ref[p] == 0:
            self.free.appendleft(p)                    # wrong: the FIFO takes freed ids at the back
        self.tables[sid][lb] = obm.NOT_RESIDENT
        host[lb] = frame


def _begin_frees_at_once(self, sid, logical):
    phys, first = begin_orig(self, sid, logical)
    for p in phys:                                     # wrong: frees before the copy completed
        self.ref[p] -= 1
        if self.ref[p] == 0:
            self.free.append(p)
        self.ref[p] += 1                               # keep the counts so finish still works
    return phys, first


def _swap_in_finish_keeps_frames(self, sid, logical):
    pend = self.pending.get(sid, {})
    for lb in logical:
        if pend.get(lb, ("",))[0] != "in":
            raise obm.InvalidArgument("nothing in flight")
    for lb in logical:
        _, p, frame = pend.pop(lb)
        self.tables[sid][lb] = p
        del self.host[sid][lb]                         # wrong: the frame never returns to the pool


begin_orig = obm.BlockManager.swap_out_begin


def test_mutant_swap_finish_fifo_front(monkeypatch):
    monkeypatch.setattr(obm.BlockManager, "swap_out_finish", _finish_to_front)
    _raises(TT.test_migration_follows_the_pages_steps)


def test_mutant_swap_frees_before_copy(monkeypatch):
    monkeypatch.setattr(obm.BlockManager, "swap_out_begin", _begin_frees_at_once)
    _raises(TT.test_migration_follows_the_pages_steps)


def test_mutant_swap_in_leaks_frames(monkeypatch):
    monkeypatch.setattr(obm.BlockManager, "swap_in_finish", _swap_in_finish_keeps_frames)
    _raises(TT.test_migration_follows_the_pages_steps)
    _raises(TT.test_random_migrations_conserve_blocks_and_frames)


# ---- FP8 storage ------------------------------------------------------------
import oracle.fp8 as ofp8  # noqa: E402
from tests import test_oracle_fp8 as T8  # noqa: E402

encode_orig = ofp8.encode
scale_orig = ofp8.scale_exponent


def _encode_ties_away(values):
    v = np.asarray(values, dtype=np.float64)
    codes = encode_orig(v)
    a = np.abs(v)
    lo = ofp8.TABLE[codes & 0x7F]
    # wrong: at an exact midpoint take the larger magnitude instead of the even code
    nxt = ofp8.TABLE[np.minimum((codes & 0x7F) + 1, 0x7E)]
    up = (a == (lo + nxt) / 2) & (nxt > lo)          # a tie that went to the smaller code
    return np.where(up, codes + 1, codes).astype(np.uint8)


def _scale_floor_rule(amax):
    if amax == 0.0:
        return 0
    return max(-127, min(127, math.frexp(float(amax))[1] - 9))   # wrong: may overflow 448


def _v_tile_no_scale(v_pool, layer, phys, head, block_size, head_dim):
    vt = v_pool[layer, phys, head]
    codes = vt[:block_size * head_dim].reshape(head_dim, block_size).T
    return ofp8.decode(codes)                                      # wrong: scale bytes ignored


def test_mutant_fp8_ties_away(monkeypatch):
    monkeypatch.setattr(ofp8, "encode", _encode_ties_away)
    _raises(T8.test_encode_matches_torch_including_ties)


def test_mutant_fp8_scale_floor(monkeypatch):
    monkeypatch.setattr(ofp8, "scale_exponent", _scale_floor_rule)
    _raises(T8.test_scale_rule_brute_force)


def test_mutant_fp8_scale_dropped(monkeypatch):
    monkeypatch.setattr(ofp8, "read_v_tile", _v_tile_no_scale)
    _raises(T8.test_decode_equals_bf16_oracle_on_representable_values)


# ---- prefix cache (oracle/radix.py) --------------------------------------------------
import oracle.radix as orx                                         # noqa: E402
from tests import test_oracle_radix as TR                          # noqa: E402

match_orig = orx.RadixCache.match
walk_orig = orx.RadixCache._walk
insert_orig = orx.RadixCache.insert


def _match_no_truncation(self, tokens):
    s_match, s_usable, blocks, handle = match_orig(self, tokens)
    return s_match, s_match, blocks, handle                        # wrong: partial tail counted


def _evict_most_recent(self, target_free):
    out = []
    while self.bm.num_free() < target_free:
        cand = self.dormant_leaves()
        if not cand:
            break
        leaf = max(cand, key=lambda n: (n.last_access, n.id))      # wrong: MRU first
        self.bm.free_blocks(leaf.block_ids)
        del leaf.parent.children[self._key(leaf.prefix_tokens, 0)]
        del self.nodes[leaf.id]
        out.append(leaf.id)
    return out


def _dormant_any(self):
    # wrong: internal nodes count as candidates (children are dropped with them)
    return [n for n in self.nodes.values() if n is not self.root and n.ref_count == 0
            and all(c.ref_count == 0 for c in n.children.values())]


def _evict_internal(self, target_free):
    out = []
    while self.bm.num_free() < target_free:
        cand = _dormant_any(self)
        if not cand:
            break
        node = min(cand, key=lambda n: (n.last_access, n.id))
        stack = [node]
        while stack:
            n = stack.pop()
            stack += list(n.children.values())
            self.bm.free_blocks(n.block_ids)
            del self.nodes[n.id]
            out.append(n.id)
        del node.parent.children[self._key(node.prefix_tokens, 0)]
    return out


def _match_no_pin(self, tokens):
    s_match, s_usable, blocks, handle = match_orig(self, tokens)
    n = self.nodes[handle]
    while n is not self.root:                                      # wrong: pins undone at once
        n.ref_count -= 1
        n = n.parent
    return s_match, s_usable, blocks, 0


def _insert_adopts_all(self, tokens, blocks):
    adopted = insert_orig(self, tokens, blocks)
    nb = min(len(blocks), len(tokens) // self.B)
    self.bm.incref([int(b) for b in blocks[:nb - adopted]])        # wrong: duplicates referenced too
    return adopted


def _walk_tail_plus_one(self, tokens):
    path, partial, pb, s_match = walk_orig(self, tokens)
    if s_match % self.B and s_match < len(tokens):
        s_match += 1                                               # wrong: one token too many
    return path, partial, pb, s_match


def _insert_split_unpinned(self, tokens, blocks):
    adopted = insert_orig(self, tokens, blocks)
    for n in self.nodes.values():                                  # wrong: split parts lose pins
        if n is not self.root and n.children and n.last_access == self.clock:
            n.ref_count = 0
    return adopted


def _fails(fn, *args):
    """The pin must fail: a failed assertion or the block manager refusing an
    operation the mutant made inconsistent."""
    with pytest.raises((AssertionError, obm.BlockManagerError)):
        fn(*args)


def test_mutant_radix_no_truncation(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "match", _match_no_truncation)
    _fails(TR.test_truncation_example)


def test_mutant_radix_mru_eviction(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "evict", _evict_most_recent)
    _fails(TR.test_lru_order, 0)


def test_mutant_radix_internal_eviction(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "evict", _evict_internal)
    _fails(TR.test_child_first)


def test_mutant_radix_match_without_pin(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "match", _match_no_pin)
    _fails(TR.test_figure6_eviction)


def test_mutant_radix_adopts_duplicates(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "insert", _insert_adopts_all)
    _fails(TR.test_brute_force_prefixes, 0, 4)


def test_mutant_radix_partial_block_off_by_one(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "_walk", _walk_tail_plus_one)
    _fails(TR.test_brute_force_prefixes, 0, 4)


def test_mutant_radix_split_drops_pins(monkeypatch):
    monkeypatch.setattr(orx.RadixCache, "insert", _insert_split_unpinned)
    _fails(TR.test_pin_counts, 0)


# ---- FP8 chunked prefill (oracle/fp8.paged_prefill) -----------------------------------
from tests import test_oracle_fp8_prefill as T8P                   # noqa: E402

fp8_prefill_orig = ofp8.paged_prefill


def _fp8_prefill_attend_before_write(q, k_new, v_new, k_pool, v_pool, layer, tables, q_start,
                                     ctx_lens, block_size, q_dtype="bf16", scale=None, chunks=None):
    import oracle.prefill as opf_
    kp, vp, _ = fp8_prefill_orig(q, k_new, v_new, k_pool, v_pool, layer, tables, q_start, ctx_lens,
                                 block_size, q_dtype, scale, chunks)
    d = q.shape[2]
    sc = att.default_scale(d) if not scale else scale
    qf, kf, vf = (layout.widen(x, q_dtype) for x in (q, k_new, v_new))
    out = np.zeros(qf.shape)
    for i in range(len(ctx_lens)):
        a, b = opf_.chunk_bounds(q_start, i)
        c = int(ctx_lens[i])
        K, V = ofp8.rebuild_sequence(k_pool, v_pool, layer, tables[i], c, block_size, d)
        # wrong: the chunk's own rows enter unquantized (attended before the write)
        out[a:b] = opf_.chunk_attention(qf[a:b], kf[a:b], vf[a:b], K, V, sc)
    return kp, vp, out


def test_mutant_fp8_prefill_attends_unquantized_chunk(monkeypatch):
    monkeypatch.setattr(ofp8, "paged_prefill", _fp8_prefill_attend_before_write)
    _raises(T8P.test_one_token_chunks_are_decode_steps)
