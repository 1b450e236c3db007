// Work protocol of the single-launch step (nest "models/qwen3-8b/files", Entries
// table, step_paged; src/attention.linnet step_paged: one QK-norm + RoPE pass over
// every token, every k/v write before any attention read, then prefill attention
// for the prompt tokens and decode attention for the rows).
//
// Written once over an environment type, so that the same control flow is the
// kernel's (step.hip, with HIP atomics and workgroup barriers) and runs on the host
// under threads that stand in for workgroups (tests/step_protocol_host.cpp).
//
// Each workgroup of the persistent grid:
//   phase 1  takes tickets from word kTicketA: ticket 0 is the tile plan, ticket
//            i >= 1 the append of chunk i - 1; after each item it publishes (word
//            kPlanDone or kAppendDone) once its writes are where every reader
//            sees them. No phase-1 item waits for
//            anything, and every ticket is taken by a running workgroup, so every
//            phase-1 item completes whatever the number of resident workgroups.
//   wait     until all append chunks and the plan have published (bounded; an
//            acquire when they have). A workgroup that gives up records the fault
//            and skips phase 2.
//   phase 2  takes tickets from word kTicketB: prefill items first, then decode
//            slices; none of them waits for another workgroup.
//   leave    the workgroup that leaves last (word kExited) clears words
//            0 .. kFault - 1 (and the GPU's append shards), so the next call
//            finds them zero.
#pragma once

namespace qknr {

// control words at the start of the step's workspace (kFault and the two words
// after it are written only when a wait gives up, and never cleared). The GPU
// counts kAppendDone in kAppendShards counters kShardStride ints apart from
// kShardBase (a workgroup adds to shard blockIdx % kAppendShards, the wait sums
// them): one counter that 264 append items add to while the finished workgroups
// poll it took about 100 us per add.
enum : int { kTicketA = 0, kAppendDone, kPlanDone, kTicketB, kExited, kFault, kSeenAppend, kSeenPlan,
             kShardBase = 64, kShardStride = 256, kAppendShards = 8,
             kCtlInts = kShardBase + kShardStride * kAppendShards };

struct StepWork {
  int n_append_items;    // phase 1: ticket 0 = the plan, tickets 1 .. n_append_items = append chunks
  int n_prefill_items;   // phase 2: tickets 0 .. n_prefill_items - 1
  int n_decode_items;    //          then n_decode_items decode slices
  int grid;              // workgroups of the launch
};

// Env provides, each called by every thread of a workgroup and returning the same
// value in every thread:
//   int  take(int word)        one atomic add of 1 to `word`; its old value
//   void publish(int word)     the workgroup's stores are complete where every
//                              workgroup reads them, then one add of 1 to
//                              `word` (the kernel's items store write-through and
//                              add relaxed; the host model adds with a release)
//   bool wait_ready(int n_append, int n_plan)
//                              until kAppendDone >= n_append and kPlanDone >=
//                              n_plan, bounded; true with an acquire when reached,
//                              false (fault recorded) when the bound ran out
//   int  leave()               one add of 1 to kExited; its old value
//   void clear()               words 0 .. kFault - 1 set to zero
//   void plan(), append(int), prefill(int), decode(int)    the items
template <class Env>
__host__ __device__ inline void run_step_protocol(Env& e, const StepWork& w) {
  for (;;) {
    const int it = e.take(kTicketA);
    if (it > w.n_append_items) break;
    if (it == 0) {
      e.plan();
    } else {
      e.append(it - 1);
    }
    e.publish(it == 0 ? kPlanDone : kAppendDone);
  }
  if (e.wait_ready(w.n_append_items, 1)) {
    for (;;) {
      const int it = e.take(kTicketB);
      if (it < w.n_prefill_items) {
        e.prefill(it);
      } else if (it - w.n_prefill_items < w.n_decode_items) {
        e.decode(it - w.n_prefill_items);
      } else {
        break;
      }
    }
  }
  if (e.leave() == w.grid - 1) e.clear();
}

}  // namespace qknr
