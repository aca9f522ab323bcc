"""The library's host table check (tg_check_tables) on the CPU: tables as
built pass, and each kind of damage a caller could do to them before they go
to the device (a page id past the pool, a page after the padding, a length
past the pages, slots reused or out of range, items that overlap or leave a
gap, group members out of order or on different pages, a page listed more
often than its reference count) is refused with TG_EINVAL and a message that
names it.  Ragged page tables and the per-(r, h) plan follow the Tangram
page, "Three mechanisms", items 2-3; shared pages the RadixAttention lesson,
"The concept"."""
import numpy as np
import pytest

from workloads import make_workload
from workloads.gen import share_arrays

tg = pytest.importorskip("non_uniform_paged_amd")


def _built(name="llama8b", group_size=0, gen=0, **over):
    w = make_workload(name, **over)
    res = tg.tg_reserve(w.head_rank, w.ratio_hi_ppm, w.ratio_lo_ppm, w.n_clusters, w.recent_ppm,
                        w.quant_block, w.n_comp, w.n_fixed, w.budget_override)
    share = None
    if w.paths is not None:
        share = tg.Share(*share_arrays(w))
    sizes = tg.tg_size_tables(res, w.page_size, w.quant_block, share, 64, 128, True, group_size, gen)
    need = sizes["pages_needed"]
    pool = tg.Pool(res.cluster_size, w.d, w.page_size, w.quant_block, [row[1] + 2 for row in need],
                   [row[0] + 2 for row in need], old_bits=w.old_bits)
    t = tg.tg_build_tables(pool, res, share, 64, 128, True, group_size, gen)
    return w, res, pool, t


def _refused(pool, res, t, fragment):
    with pytest.raises(tg.TGError) as e:
        tg.tg_check_tables(pool, res, t)
    assert e.value.name == "TG_EINVAL"
    assert fragment in str(e.value), str(e.value)


@pytest.mark.parametrize("name,gs,gen,over", [
    ("tiny", 0, 0, {}), ("llama8b", 0, 0, dict(B=6)), ("ragged", 0, 0, dict(B=8)),
    ("tiered", 0, 0, dict(B=2, ctx=("fixed", 3000))), ("tiered4", 0, 0, dict(B=2, ctx=("fixed", 3000))),
    ("radix", 8, 0, dict(B=24, share=dict(prefix=300, branch=80, n_branches=3, suffix=(8, 300)))),
    ("llama8b", 0, 200, dict(B=4)), ("tiered", 0, 500, dict(B=2, ctx=("fixed", 3000))),
])
def test_built_tables_pass(name, gs, gen, over):
    w, res, pool, t = _built(name, gs, gen, **over)
    tg.tg_check_tables(pool, res, t)


def test_page_past_capacity():
    w, res, pool, t = _built(B=4)
    t.bt[0][1][1, 0] = pool.capacity(0, 1)
    _refused(pool, res, t, "past the capacity")


def test_page_after_padding():
    w, res, pool, t = _built(B=4)
    row = t.bt[0][1][0]
    assert int((row >= 0).sum()) >= 2
    row[0] = -1  # a hole: the row's other pages now follow its padding
    _refused(pool, res, t, "after the row's last page")


def test_page_listed_beyond_its_refcount():
    w, res, pool, t = _built(B=4)
    t.bt[0][1][1, 0] = t.bt[0][1][0, 0]  # a private page now in two rows
    _refused(pool, res, t, "reference count")


def test_length_past_pages():
    w, res, pool, t = _built(B=4)
    row = t.bt[0][1][0]
    t.len[0, 0, 1] = int((row >= 0).sum()) * 16 + 16
    h0 = int(np.where(np.array(res.cluster_of_head) == 0)[0][0])
    t.len[0, h0, 1] = int((row >= 0).sum()) * 16 + 1
    _refused(pool, res, t, "passes its pages")


def test_int8_length_not_whole_blocks():
    w, res, pool, t = _built("tiered", B=2, ctx=("fixed", 3000))
    t.len[0, 0, 0] -= 1
    _refused(pool, res, t, "len of (0, 0)")


def test_part_off_decreasing():
    w, res, pool, t = _built(B=4)
    t.part_off[3] = t.part_off[2] - 1
    _refused(pool, res, t, "part_off decreases")


def test_slot_used_twice():
    w, res, pool, t = _built(B=4)
    plan = t.plan
    # two items of one (r, h) with their slots made equal
    r, h = int(plan[0, 0]), int(plan[0, 1])
    same = [k for k in range(1, len(plan)) if plan[k, 0] == r and plan[k, 1] == h]
    assert same, "the test needs a pair with two items"
    plan[same[0], 5] = plan[0, 5]
    _refused(pool, res, t, "used twice")


def test_slot_of_another_pair():
    w, res, pool, t = _built(B=4)
    plan = t.plan
    plan[0, 5] = (int(plan[0, 5]) + t.part_off[-1] // 2) % t.part_off[-1]
    _refused(pool, res, t, "outside")


def test_items_overlap_and_gap():
    w, res, pool, t = _built(B=4)
    plan = t.plan
    r, h, tier = int(plan[0, 0]), int(plan[0, 1]), int(plan[0, 2])
    k = [i for i in range(len(plan)) if (plan[i, 0], plan[i, 1], plan[i, 2]) == (r, h, tier) and plan[i, 3] > 0][0]
    saved = int(plan[k, 3])
    plan[k, 3] = saved - 16  # overlaps the item before it
    _refused(pool, res, t, "covered twice")
    plan[k, 3] = saved + 16  # leaves a gap
    _refused(pool, res, t, "uncovered")


def test_items_end_before_live_rows():
    w, res, pool, t = _built(B=4)
    plan = t.plan
    # the last item of a pair's bf16 range cut one page short
    r, h = 0, 0
    ks = [i for i in range(len(plan)) if (plan[i, 0], plan[i, 1], plan[i, 2]) == (r, h, 1)]
    last = max(ks, key=lambda i: plan[i, 4])
    if plan[last, 4] - plan[last, 3] <= 16:
        pytest.skip("item too short to cut")
    plan[last, 4] -= 16
    _refused(pool, res, t, "rows are live")


def test_group_members_out_of_order_and_on_other_pages():
    w, res, pool, t = _built("radix", 8, B=24, share=dict(prefix=300, branch=80, n_branches=3, suffix=(8, 300)))
    assert t.n_gitems > 0
    gm = t.gitems[0]
    assert gm[1, 0] >= 0
    saved = gm[:2].copy()
    gm[[0, 1]] = gm[[1, 0]]
    _refused(pool, res, t, "not ascending")
    gm[:2] = saved
    tg.tg_check_tables(pool, res, t)
    # a member's first shared page replaced by a private one of another row
    h = int([row for row in t.plan if row[0] == -1][0][1])
    c = int(res.cluster_of_head[h])
    r1 = int(gm[1, 0])
    t0 = int([row for row in t.plan if row[0] == -1][0][3])
    bt = t.bt[c][1]
    priv = int(bt[r1, np.where(bt[r1] >= 0)[0][-1]])
    bt[r1, t0 // 16] = priv
    with pytest.raises(tg.TGError) as e:
        tg.tg_check_tables(pool, res, t)
    assert "differs" in str(e.value) or "reference count" in str(e.value), str(e.value)


def test_group_item_missing_from_plan():
    w, res, pool, t = _built("radix", 8, B=24, share=dict(prefix=300, branch=80, n_branches=3, suffix=(8, 300)))
    plan = t.plan
    k = [i for i in range(len(plan)) if plan[i, 0] == -1][0]
    plan[k, 0] = -2 if t.n_gitems > 1 else -1  # now group item 1 twice, group item 0 never
    _refused(pool, res, t, "group item")


def test_request_count_must_match():
    w, res, pool, t = _built(B=4)
    t.struct.B = 3
    _refused(pool, res, t, "requests")
