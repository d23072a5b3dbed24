"""CPU model of the claim queues and of the claim entries that carry a claimed item from
a workgroup's controller wave to its worker waves (section "Tasks": the drain tasks of
the shared work queue; ATTN and MoE-up claimers).  The rules are those of the kernel:

- attention: claimer i of n takes item i first, with no atomic; later items come from
  n + (fetch-and-add on the queue head);
- MoE-up, queue mode: claimer i >= n_attn takes item i - n_attn first (n_free of them); the
  others, and every later claim, take n_free + (fetch-and-add);
- MoE-up, static mode: free claimer f takes items f, f + n_free, ...; claimers with an
  attention item take none;
- a claimer stops at the first item >= n_items.

Under random interleavings of the claimers' atomics every item is processed exactly once
and every claimer stops.  The claim entries: the controller stores each claimed item with
its task index into one of two LDS slots before a barrier, the workers read it after; a
claimer loop ends without a further barrier, so the controller may already have stored
the first entry of its next claimer task when a slower worker reads its last entry of
this one.  With the task index in the entry every worker of every task sees exactly the
controller's item sequence; without it (the kernel's earlier form) some interleaving
makes a worker take the next task's item.  CPU only."""
import itertools
import random

import pytest

END = 1 << 30


def run_queue(first, base, n_items, n_cl, rng):
    """first[i]: claimer i's first item (None: claim from the queue); returns the item
    lists per claimer, under a random order of the claimers' fetch-and-adds."""
    head = 0
    cur = [f if f is not None else None for f in first]
    need_claim = [f is None for f in first]
    items = [[] for _ in range(n_cl)]
    active = list(range(n_cl))
    atomics = 0
    while active:
        i = rng.choice(active)
        if need_claim[i]:
            cur[i] = base + head
            head += 1
            atomics += 1
        if cur[i] >= n_items:
            active.remove(i)
            continue
        items[i].append(cur[i])
        need_claim[i] = True
    return items, atomics


def check_exactly_once(items, n_items):
    flat = sorted(x for lst in items for x in lst)
    assert flat == list(range(n_items))


@pytest.mark.parametrize("seed", range(20))
def test_attention_queue_exactly_once(seed):
    rng = random.Random(seed)
    n_cl, n_items = rng.randint(1, 40), rng.randint(0, 120)
    items, atomics = run_queue(list(range(n_cl)), n_cl, n_items, n_cl, rng)
    check_exactly_once(items, n_items)
    assert atomics <= max(0, n_items - n_cl) + n_cl


@pytest.mark.parametrize("seed", range(20))
def test_moe_queue_mode_exactly_once(seed):
    rng = random.Random(100 + seed)
    n_cl = rng.randint(1, 40)
    n_attn = rng.randint(0, n_cl)
    n_free, n_items = n_cl - n_attn, rng.randint(0, 150)
    first = [i - n_attn if i >= n_attn else None for i in range(n_cl)]
    items, _ = run_queue(first, n_free, n_items, n_cl, rng)
    check_exactly_once(items, n_items)


@pytest.mark.parametrize("n_cl,n_attn,n_items", [(256, 36, 512), (256, 200, 1856), (7, 0, 3), (5, 5, 0)])
def test_moe_static_mode_exactly_once(n_cl, n_attn, n_items):
    n_free = n_cl - n_attn
    items = [list(range(ci - n_attn, n_items, n_free)) if ci >= n_attn and n_free else [] for ci in range(n_cl)]
    if n_free:
        check_exactly_once(items, n_items)
    # the largest share differs from the smallest by at most one item
    shares = [len(x) for x in items[n_attn:]]
    assert not shares or max(shares) - min(shares) <= 1


def _entry_protocol(tagged, tasks, schedule):
    """One workgroup running claimer tasks back to back.  tasks[t] = the item sequence the
    controller claims in task t (ending with END).  The controller stores entry k = j & 1
    of task t (item, t) before the barrier that ends iteration j - 1 (entry 0 before the
    task's first barrier); every wave reads entry j & 1 after that barrier.  After a task's
    last barrier the controller starts the next task at once; schedule[t] says whether the
    slow worker reads its last entry of task t before (0) or after (1) the controller's
    first store of task t + 1.  Returns the item sequences the worker saw, per task."""
    entry = [(None, None), (None, None)]
    seen = []
    for t, seq in enumerate(tasks):
        entry[0] = (seq[0], t)
        got = []
        for j, item in enumerate(seq):
            if j + 1 < len(seq):
                entry[(j + 1) & 1] = (seq[j + 1], t)
            last = item >= END
            if last and t + 1 < len(tasks) and schedule[t] == 1:
                # the controller has left the task and stored its next task's first entry
                pending = (tasks[t + 1][0], t + 1)
                if (j & 1) == 0:
                    entry[0] = pending
            v, tag = entry[j & 1]
            w = v if (not tagged or tag == t) else END
            got.append(w)
            if w >= END:
                break
        seen.append(got)
    return seen


@pytest.mark.parametrize("tagged", [True, False])
def test_claim_entries_need_the_task_tag(tagged):
    # claimer tasks whose item sequences end at an even or an odd iteration
    task_sets = [[[3, 7, END], [5, END], [2, 4, 6, END]], [[1, END], [8, 9, END]], [[END], [0, END]]]
    failures = 0
    for tasks in task_sets:
        for schedule in itertools.product((0, 1), repeat=len(tasks) - 1):
            seen = _entry_protocol(tagged, tasks, list(schedule) + [0])
            for t, seq in enumerate(tasks):
                if seen[t] != seq[:len(seen[t])] or seen[t][-1] < END:
                    failures += 1
    if tagged:
        assert failures == 0
    else:
        assert failures > 0, "the model no longer shows the hazard the tag removes"
