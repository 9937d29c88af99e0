"""The n-gram drafter against hand-built sequences, one per rule it follows
([k3_run.c] --spec / spec_draft(): match length 4 then 3, every occurrence
must agree, stop where continuations diverge, at most 8 drafts)."""
from quantized_gemv_gqa_decode_amd.draft import MAX_DRAFT, ngram_draft


def test_no_earlier_occurrence_no_draft():
    assert ngram_draft([1, 2, 3, 4, 5, 6, 7, 8, 9], 8) == []
    assert ngram_draft([1, 2, 3], 8) == []                   # shorter than any n-gram + 1
    assert ngram_draft([5, 5, 5, 5, 5, 5], 0) == []          # nothing asked for


def test_single_occurrence_copies_what_followed():
    # the 4-gram 1 2 3 4 occurred once; what followed it, up to the sequence end
    assert ngram_draft([1, 2, 3, 4, 5, 6, 1, 2, 3, 4], 8) == [5, 6, 1, 2, 3, 4]
    assert ngram_draft([1, 2, 3, 4, 5, 6, 1, 2, 3, 4], 2) == [5, 6]


def test_at_most_eight():
    seq = list(range(100, 120)) + list(range(100, 104))
    d = ngram_draft(seq, 32)
    assert len(d) == MAX_DRAFT == 8
    assert d == list(range(104, 112))


def test_two_occurrences_stop_where_they_diverge():
    # occurrences at 0 and 7; both continue 7 8, then 9 vs 5
    seq = [1, 2, 3, 4, 7, 8, 9, 1, 2, 3, 4, 7, 8, 5, 1, 2, 3, 4]
    assert ngram_draft(seq, 8) == [7, 8]


def test_every_occurrence_must_agree_not_only_the_two_latest():
    # three occurrences of 1 2 3 4: the two most recent continue 7 8 ..., the
    # oldest 7 9: the draft stops after 7 (the stated rule covers every one)
    seq = [1, 2, 3, 4, 7, 9, 0, 1, 2, 3, 4, 7, 8, 0, 1, 2, 3, 4, 7, 8, 0, 1, 2, 3, 4]
    assert ngram_draft(seq, 8) == [7]


def test_disagreeing_4gram_falls_back_to_3gram():
    # 4-gram 9 1 2 3 occurs twice with different next ids (4 vs 5): no draft
    # at n = 4; the 3-gram 1 2 3 has a third, later occurrence (after 6) whose
    # continuation agrees with no one... so build it to agree: all three
    # 3-gram occurrences are followed by 4 except those of the 4-gram
    seq = [9, 1, 2, 3, 4, 9, 1, 2, 3, 5, 6, 1, 2, 3, 4, 9, 1, 2, 3]
    # n = 4: suffix 9 1 2 3 occurs at 0 (-> 4) and 5 (-> 5): disagree, empty
    # n = 3: suffix 1 2 3 occurs at 1 (-> 4 9 1 2 3 5 ...), 6 (-> 5), 11 (-> 4)
    #        the occurrence at 6 disagrees at once: empty as well
    assert ngram_draft(seq, 8) == []
    seq2 = [7, 1, 2, 3, 4, 9, 1, 2, 3, 5, 6, 1, 2, 3, 4, 8, 9, 1, 2, 3]
    # n = 4: 9 1 2 3 occurs only at 5 (-> 5 6 1 2 3 4 8 ...): draft from it
    assert ngram_draft(seq2, 3) == [5, 6, 1]
    seq3 = [6, 1, 2, 3, 4, 5, 8, 8, 1, 2, 3, 4, 5, 7, 1, 2, 3]
    # n = 4: 7 1 2 3 never occurred earlier; n = 3: 1 2 3 at 1 and 8, both -> 4 5, then 8 vs 7
    assert ngram_draft(seq3, 8) == [4, 5]


def test_overlapping_occurrence_of_a_repeated_token():
    # 5 5 5 5 5: the suffix 4-gram occurs at 0 (continuation 5) -- overlapping
    assert ngram_draft([5, 5, 5, 5, 5], 8) == [5]
    # the most recent occurrence (at 7) is followed by one token before the
    # sequence ends: the draft copies only what followed it
    assert ngram_draft([5] * 12, 8) == [5]
