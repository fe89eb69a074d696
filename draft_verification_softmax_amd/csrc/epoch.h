// epoch.h -- the call epoch of a workspace and the arrival that ends a call.
//
// Workgroups of one call exchange 64-bit words whose high half is the call's tag, the
// workspace epoch plus one; a word with any other tag is absent.  The epoch advances when
// the last unit of the call arrives, and every workgroup that reads the epoch does so before
// its unit arrives, unless a bounded wait of the call gave up: then a workgroup may still
// be on its way and read the advanced epoch, and the words it writes would carry the next
// call's tag.  So the arrival that ends such a call stores the tag with the poison bit set.
// A workgroup of a verification or sampling call that reads a poisoned epoch writes nothing
// that another call reads (members return; the finalize writes "nothing verified" outputs
// and raises a device error flag), until the workspace is zero-filled again.  The same
// happens once the tags are spent (2^31 - 1 calls on one workspace).
//
// Plain C++ (no HIP types): the arithmetic and the arrival below also build with a host
// compiler, for the CPU tests.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SV_HD __host__ __device__
#else
#define SV_HD
#endif

namespace sv {

constexpr uint32_t kEpochPoison = 0x80000000u;   // set in the epoch of a workspace that verifies nothing

SV_HD constexpr bool epoch_poisoned(uint32_t epoch) { return (epoch & kEpochPoison) != 0u; }

// The tag of the call that reads `epoch`.
SV_HD constexpr uint32_t epoch_tag(uint32_t epoch) { return epoch + 1u; }

// The epoch the arrival that ends a call stores: the call's tag, poisoned when a wait of the
// call gave up (`gave_up`) or when the next tag would reach the poison bit.
SV_HD constexpr uint32_t epoch_after(uint32_t tag, bool gave_up) {
    return (gave_up || tag >= kEpochPoison - 1u) ? (tag | kEpochPoison) : tag;
}

// An arrival counter counts in its low 31 bits; an arrival that gave up a wait first sets
// bit 31 (sticky: an or, then its add, both on the same word, so the add that completes the
// counter returns the bit whenever any unit on it gave up).
constexpr uint32_t kArriveGaveUp = 0x80000000u;

struct Arrival {
    bool last;      // this arrival completes the call
    bool gave_up;   // (last only) some arrival of the call gave up a wait
};

// Arrival of unit i of n (one call per unit) at the end of a call; `last` is true for exactly
// one unit, whose arrival completes the call.  Up to `single` units share the second-level
// counter `top` directly.  More land on `slots_max` first-level counters `slot_ctr(s)`
// (i modulo the slot count); the arrival that fills a slot moves on to `top`, carrying
// whether a unit of its slot gave up.  Each counter is back at zero once it is full.
// add(p, v) and or_(p, v) are returning atomics on a uint32 counter, zero(p) an atomic store
// of 0.
template <class Ctr, class SlotCtr, class Add, class Or, class Zero>
SV_HD inline Arrival arrive(int64_t i, int64_t n, bool gave_up, Ctr *top, SlotCtr slot_ctr, int single, int slots_max,
                            Add add, Or or_, Zero zero) {
    auto one = [&](Ctr *c, bool g) -> uint32_t {
        if (g) or_(c, kArriveGaveUp);
        return add(c, 1u);
    };
    if (n <= single) {
        const uint32_t old = one(top, gave_up);
        if ((old & ~kArriveGaveUp) != (uint32_t)(n - 1)) return Arrival{false, false};
        zero(top);
        return Arrival{true, (old & kArriveGaveUp) != 0u};
    }
    const int slot = (int)(i % slots_max);
    const int in_slot = (int)((n - 1 - slot) / slots_max) + 1;   // units i < n on this slot
    const int slots = (int)(n < slots_max ? n : slots_max);
    Ctr *c = slot_ctr(slot);
    const uint32_t old = one(c, gave_up);
    if ((old & ~kArriveGaveUp) != (uint32_t)(in_slot - 1)) return Arrival{false, false};
    zero(c);
    const uint32_t old2 = one(top, (old & kArriveGaveUp) != 0u);
    if ((old2 & ~kArriveGaveUp) != (uint32_t)(slots - 1)) return Arrival{false, false};
    zero(top);
    return Arrival{true, (old2 & kArriveGaveUp) != 0u};
}

}  // namespace sv
