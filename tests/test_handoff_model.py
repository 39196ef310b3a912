"""Exhaustive host model of the one-launch decode path's hand-off of T.

The workgroups of one launch exchange their rows of T through tagged entries
in the workspace: each reads the epoch E, stores its entries tagged E + 1 and
polls, bounded, until every entry carries E + 1.  The model explores every
interleaving of those steps (a workgroup may start only after others have
finished: the GPU held by other work) over consecutive calls on one
workspace, with per-entry poll reads, a bounded number of poll passes, and a
workgroup free to give up after any failed pass.  It checks that

  * no workgroup ever accepts an entry written by an earlier call (its rows
    of Y would be silently wrong), and
  * after every call each tag ever written is at most the epoch.

The kernels' protocol (every workgroup that gives up, and workgroup 0 once
it has seen every entry, raise the epoch to their tag by an atomic max) keeps
both.  The earlier protocol, where only workgroup 0 advanced the epoch and
only on success, breaks the first: the model finds the interleaving where
workgroup 0 gives up before a late workgroup publishes, and the next call
accepts that late entry.  This runs on the CPU only; no GPU is involved."""
import pytest

START, PUB, POLL, FIN, DONE = range(5)


def explore(P, calls, passes, protocol):
    """Depth-first search over every reachable state.  Returns a list of
    violations found (empty if none)."""
    violations = []
    # global state: (call, epoch, tags, vals, locals); a local is
    # (pc, E, i, npass, match, stale, ok)
    init_local = (START, 0, 0, 0, True, False, False)
    start = (0, 0, (0,) * P, (-1,) * P, (init_local,) * P)
    seen = set()
    stack = [start]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        call, epoch, tags, vals, locs = st
        if call == calls:
            continue
        if all(l[0] == DONE for l in locs):
            if any(t > epoch for t in tags):
                violations.append(("tag above epoch after call", call, epoch, tags))
            stack.append((call + 1, epoch, tags, vals, (init_local,) * P))
            continue
        for w in range(P):
            pc, E, i, npass, match, stale, ok = locs[w]
            nt, nv, ne = list(tags), list(vals), epoch
            succ = []
            if pc == START:
                succ.append((PUB, epoch, 0, 0, True, False, False))
            elif pc == PUB:
                nt[w], nv[w] = E + 1, call
                succ.append((POLL, E, 0, 0, True, False, False))
            elif pc == POLL:
                hit = tags[i] == E + 1
                m2 = match and hit
                s2 = stale or (hit and vals[i] != call)
                if i + 1 < P:
                    succ.append((POLL, E, i + 1, npass, m2, s2, False))
                elif m2:
                    if s2:
                        violations.append(("accepted a stale entry", call, w, tags, vals))
                    succ.append((FIN, E, 0, npass, True, s2, True))
                else:
                    succ.append((FIN, E, 0, npass, False, False, False))          # give up now
                    if npass + 1 < passes:
                        succ.append((POLL, E, 0, npass + 1, True, False, False))  # poll again
            elif pc == FIN:
                want = E + 1
                if protocol == "atomic_max":
                    if not ok or w == 0:
                        ne = max(epoch, want)
                elif protocol == "first_stores_on_success":
                    if ok and w == 0:
                        ne = want
                else:
                    raise ValueError(protocol)
                succ.append((DONE, E, 0, 0, True, False, ok))
            else:
                continue
            for nl in succ:
                l2 = list(locs)
                l2[w] = nl
                stack.append((call, ne, tuple(nt), tuple(nv), tuple(l2)))
        if len(violations) > 8:
            break
    return violations, len(seen)


@pytest.mark.parametrize("P,calls,passes", [(2, 3, 2), (3, 2, 2), (2, 4, 1)])
def test_protocol_never_accepts_stale_entries(P, calls, passes):
    violations, states = explore(P, calls, passes, "atomic_max")
    assert states > 100
    assert violations == [], violations[:3]


def test_model_finds_the_defect_of_the_earlier_protocol():
    """The model is not vacuous: with only workgroup 0 advancing the epoch on
    success, a give-up lets a later call accept a stale entry."""
    violations, _ = explore(2, 2, 1, "first_stores_on_success")
    assert any(v[0] == "accepted a stale entry" for v in violations)
