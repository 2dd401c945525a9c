// ring.hpp -- the stage-ring schedule of the pipelined mainloop.
//
// The "B200 TMA Pipeline Designer" page (Executable steps 6 and 7) describes a
// ring of PIPE_DEPTH shared-memory stages with ready/free synchronisation and a
// three-phase timeline: a prologue that fills the first stages, a steady state
// that overlaps the load of a later K tile with the compute of the current one,
// and an epilogue that stops issuing loads and drains.  On gfx950 the "ready"
// signal is each wave's own s_waitcnt vmcnt on the direct-to-LDS loads it
// issued, followed by the workgroup s_barrier; the same barrier is the "free"
// signal for the slot whose reads every wave has finished (each wave drains its
// LDS reads with s_waitcnt lgkmcnt(0) before arriving).
//
// The ring is counted in operand slots: U = 2*PIPE_DEPTH + HALF slots, where
// HALF = 1 adds one slot beyond whole stages.  The K loop consumes a sequence
// of units, unit 2t being the A tile and unit 2t+1 the B tile of K tile t, and
// unit s lives in slot s % U.  (With U even this is the classic ring of U/2
// stages, A in the even slots and B in the odd ones.)
//
// Spread rings (U >= 5):
//   prologue : issue units 0 .. U-3
//              wait(units 0, 1); barrier; read fragments of tile 0, first k-step
//   tile t   : the barrier that made tile t ready also freed the slots of tile
//              t-1; refill them with units 2t+U-2 and 2t+U-1 by loads spread
//              over tile t's k-steps, computing all but its last k-step
//              (reading ahead one k-step);
//              wait(unit 2t+3, i.e. B(t+1))  -- the U-4 newer units may stay
//                                                 in flight
//              barrier  -- tile t+1 ready for every wave, and every wave has
//                          finished reading tile t
//              read fragments of tile t+1, first k-step
//              compute the last k-step of t (operands already in registers)
//   epilogue : wait for everything (the trailing units, past the last tile,
//              are out of range and land as zeros).
// The loop body is unrolled by the ring period so that every slot is a
// constant; the tiles of a last, partial period run after the loop, each
// under its own test, so no tile past KT is computed.
// With U = 2D the refill during tile t is tile t+D-1, as in a stage ring; with
// U = 5 (two and a half 64-deep stages of a 256 x 256 tile fit in 160 KB) the
// refill is B(t+1) and A(t+2): B gets one tile of compute to land, A two.
//
// Two-stage ring (U = 4, burst): tiles 0, 1 issued up front; after the barrier
// that frees tile t's stage, tile t+2 is issued into it at once:
//   prologue : issue tiles 0 .. min(D, KT)-1
//              wait(tile 0); barrier; read fragments of tile 0, first k-step
//   tile t   : compute all but the last k-step of t (reading ahead one k-step)
//              if t+1 < KT:
//                 wait(tile t+1)   -- vmcnt allows inflight(t+1) later tiles
//                 barrier          -- tile t+1 ready for every wave, and every
//                                     wave has finished reading tile t
//                 if t+D < KT: issue tile t+D into the stage of tile t
//                 read fragments of tile t+1, first k-step
//              compute the last k-step of t (operands already in registers)
//
// D == 1 has a single stage, so the next tile can only be issued after the
// barrier that frees it, and must be waited for at once (no overlap); it is
// kept as the no-pipelining baseline.
//
// The two-stage and whole-stage forms pad the K loop to a whole number of
// ring periods with tiles whose loads are all out of range (they land as
// zeros).
#pragma once

#if defined(__HIPCC__)
#define IGC_HD __host__ __device__
#else
#define IGC_HD
#endif

namespace igc {

struct Ring {
    // Two-stage ring: tiles issued before the wait for tile t.
    IGC_HD static constexpr int issued_before_wait(int D, int KT, int t) {
        return ((t > 1 ? t - 1 : 0) + D) < KT ? ((t > 1 ? t - 1 : 0) + D) : KT;
    }
    // Two-stage ring: tiles newer than t that may still be in flight when tile
    // t must have landed; the wave's vmcnt is this times its loads per tile.
    IGC_HD static constexpr int inflight_after(int D, int KT, int t) {
        return issued_before_wait(D, KT, t) - 1 - t;
    }
    // Operand slots of a ring of D stages plus HALF extra slot.
    IGC_HD static constexpr int units(int D, int half) { return 2 * D + half; }
    // Rings of five or more operand slots refill the slots freed at a barrier
    // during the next tile's k-steps (loads interleaved with the MFMAs);
    // smaller rings issue the refill right after the barrier.
    IGC_HD static constexpr bool spread(int U) { return U >= 5; }
    // Slot of unit s.
    IGC_HD static constexpr int slot_of(int U, int s) { return s % U; }
    // Tiles after which the slot pattern repeats (tile t uses slots 2t%U and
    // (2t+1)%U): U for an odd ring, U/2 for an even one.
    IGC_HD static constexpr int period(int U) { return U % 2 ? U : U / 2; }
    // Spread rings: units newer than B(t+1) allowed in flight at its wait, and
    // the loads (per wave) they make when A and B units take ipw_a and ipw_b
    // wave instructions; the first of them is an A unit.
    IGC_HD static constexpr int wait_units(int U) { return U - 4; }
    IGC_HD static constexpr int wait_loads(int U, int ipw_a, int ipw_b) {
        return (U - 3) / 2 * ipw_a + (U - 4) / 2 * ipw_b;
    }
};

}  // namespace igc
