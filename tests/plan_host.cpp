// Host build of the grouped-GEMM tile planner for the CPU coverage checks
// (tests/test_plan_coverage.py): the functions of the library's own
// plan.hpp, which its device planner runs too, behind a C interface.
#include "plan.hpp"

namespace P = moe::plan;

extern "C" {

// Split flag and workgroup slots of a 256x256-tile launch, as the library's
// launcher sizes them (pairs: short segments may take tile pairs, the 8-wave
// kernel's plan; 0 for the 4-wave kernel).
int moe_plan_slots(int E, int rows, int shared_M, int Nr, int Kr, int Ns, int Ks, int pairs,
                   int* split) {
  P::Shape s{E, rows, shared_M, Nr, Kr, Ns, Ks, 0, 0, pairs};
  s.split = P::split_ok(s) ? 1 : 0;
  *split = s.split;
  return P::launch_slots<256, 256>(s);
}

// The launch's whole tile table: (slots + reduce slots) entries of 16 ints.
void moe_plan_table(const int32_t* offsets, int E, int rows, int shared_M, int Nr, int Kr, int Ns,
                    int Ks, int split, int slots, int pairs, int* table) {
  const P::Shape s{E, rows, shared_M, Nr, Kr, Ns, Ks, split, slots, pairs};
  P::plan_table_serial<256, 256, P::kBlockCols>(s, offsets, table);
}

int moe_plan_reduce_slots() { return P::kReduceSlots; }
int moe_plan_entry_ints() { return P::kEntryInts; }

}  // extern "C"
