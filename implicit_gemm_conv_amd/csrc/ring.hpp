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
// Schedule for D = PIPE_DEPTH >= 2 and KT K tiles (tile t lives in slot t % D):
//
//   prologue : issue tiles 0 .. min(D, KT)-1
//              wait(tile 0); barrier; read fragments of tile 0, first k-step
//   tile t   : compute all but the last k-step of t (reading ahead one k-step)
//              if t+1 < KT:
//                 wait(tile t+1)   -- vmcnt allows inflight(t+1) later tiles
//                 barrier          -- tile t+1 ready for every wave, and every
//                                     wave has finished reading tile t
//                 if t+D < KT: issue tile t+D into slot t % D  (just freed)
//                 read fragments of tile t+1, first k-step
//              compute the last k-step of t (operands already in registers)
//   epilogue : nothing left in flight; accumulators go to the output.
//
// D >= 3 ("spread" rings): the prologue issues tiles 0 .. D-2 only; after the
// barrier before tile t, the slot of tile t-1 is free and is refilled with tile
// t+D-1 by loads interleaved through tile t's k-steps.  Every wait then allows
// exactly D-2 newer tiles in flight.
//
// D == 1 has a single slot, so the next tile can only be issued after the
// barrier that frees it, and must be waited for at once (no overlap); it is
// kept as the no-pipelining baseline.
//
// In both pipelined forms the K loop is padded to a multiple of D with tiles
// whose loads are all out of range (they land as zeros).
#pragma once

#if defined(__HIPCC__)
#define IGC_HD __host__ __device__
#else
#define IGC_HD
#endif

namespace igc {

struct Ring {
    // Tiles issued before the wait for tile t (D >= 2).
    IGC_HD static constexpr int issued_before_wait(int D, int KT, int t) {
        return ((t > 1 ? t - 1 : 0) + D) < KT ? ((t > 1 ? t - 1 : 0) + D) : KT;
    }
    // Tiles newer than t that may still be in flight when tile t must have
    // landed (D >= 2): the wave's vmcnt is this times its loads per tile.
    IGC_HD static constexpr int inflight_after(int D, int KT, int t) {
        return issued_before_wait(D, KT, t) - 1 - t;
    }
    IGC_HD static constexpr int slot(int D, int tile) { return tile % D; }
    // Rings of three or more stages refill the slot freed at a barrier during
    // the next tile's k-steps (loads interleaved with the MFMAs); two-stage
    // rings issue the refill right after the barrier.
    IGC_HD static constexpr bool spread(int D) { return D >= 3; }
    IGC_HD static constexpr int prologue_tiles(int D, int KT) { return D < KT ? D : KT; }
};

}  // namespace igc
